// pkv_attn.hip -- attention forward kernels for gfx950.
//
// What is computed (per request r, query token t, head h):
//   out = softmax_j(scale * q . k_j) v_j over the keys j the query may see,
//   lse = log sum_j exp(scale * q . k_j)
// with the packed-batch semantics of "How vLLM attention kernels handle
// multiple requests in parallel": requests are isolated (sections 1 and 5),
// the causal mask comes from request-local positions and is bottom-right
// aligned when the request has cached context (sections 4 and 10), keys are
// found through the block table (section 11), the score tile lives only in
// registers and is folded into the output by the online softmax (sections 6
// and 7), and long KV ranges can be split over workgroups whose partial
// results a second kernel merges by log-sum-exp (section 12).
//
// Kernels:
//  decode_kernel   one work item = (request, kv head, KV split); the q_len x g
//                  query rows of a GQA group (<= 16) are the columns of a
//                  16x16x32 bf16 MFMA, so one K/V load serves the whole group.
//                  Four waves share the item's key range; K goes straight from
//                  HBM into MFMA registers, V is staged in LDS and read back
//                  transposed; the waves merge their states through LDS.
//  prefill_kernel  one work item = (request, kv head, 128 query rows, KV split);
//                  rows are (token, head-of-group) pairs, 32 per wave, on
//                  32x32x16 bf16 MFMA; K/V tiles are staged in LDS for all
//                  four waves; tiles entirely in a wave's future are skipped
//                  and only tiles crossing the diagonal build a per-element mask.
//  generic_kernel  one wave per (token, head); plain fp32 arithmetic on the
//                  vector ALUs for fp32 inputs and head sizes without an MFMA
//                  instantiation.
//  combine_kernel  log-sum-exp merge of the split partials.
//  merge_kernel    merge of two attention states (cascade prefix / suffix).
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

// 16 bytes of K or V for one row: 8 bf16 values (fp8 caches are widened; exact).
template <bool FP8>
__device__ __forceinline__ u32x4 load_kv8(const void* base, int64_t elem) {
    if constexpr (FP8) {
        return fp8x8_to_bf16x8(*(const u32x2*)((const uint8_t*)base + elem));
    } else {
        return *(const u32x4*)((const uint16_t*)base + elem);
    }
}

// ----------------------------------------------------------------- decode

template <int HD, bool FP8>
__global__ __launch_bounds__(256) void decode_kernel(FwdParams p) {
    constexpr int TILE = kDecodeTile;
    constexpr int NW = kDecodeWaves;
    constexpr int KS = HD / 32;             // k-steps of S^T = K Q^T
    constexpr int MB = HD / 16;             // 16-row blocks of O^T
    constexpr int VP = HD + 16;             // LDS pitch of a V row (bf16 elements)
    constexpr int CPR = HD / 8;             // 16-byte chunks per row
    constexpr int VLOADS = TILE * CPR / 64; // V chunks per lane per tile
    static_assert(HD % 32 == 0 && VLOADS >= 1, "");
    constexpr int VSM = NW * TILE * VP;     // bf16 elements of V staging
    constexpr int OSM = NW * 16 * HD * 2;   // the same bytes reused as fp32 partial outputs
    __shared__ __attribute__((aligned(16))) uint16_t smem[VSM > OSM ? VSM : OSM];
    __shared__ float sm_m[NW][16], sm_l[NW][16];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int s = blockIdx.x, kh = blockIdx.y, r = blockIdx.z;
    const int q0 = p.qsl[r];
    const int q_len = p.qsl[r + 1] - q0;
    if (q_len <= 0) return;
    const int L = p.seq_lens ? p.seq_lens[r] : q_len;
    const int ctx = L - q_len;
    const int k_begin = p.num_splits > 1 ? s * p.split_len : 0;
    const int k_end = p.num_splits > 1 ? min(L, k_begin + p.split_len) : L;
    if (k_begin >= k_end) return;  // no row of this item sees a key here; the merge never reads it

    const int g = p.g;
    const int row = lane & 15;
    const int G = lane >> 4;
    const int rows_total = q_len * g;
    const bool row_ok = row < rows_total;
    const int tl = row_ok ? row / g : 0;
    const int hh = kh * g + (row_ok ? row % g : 0);
    int limit = p.causal ? min(L, ctx + tl + 1) : L;
    limit = row_ok ? min(limit, k_end) : 0;

    u32x4 qf[KS];
    {
        const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(q0 + tl) * p.H + hh) * HD + G * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? *(const u32x4*)(qp + ks * 32) : u32x4{0u, 0u, 0u, 0u};
    }
    float sl2 = p.scale_log2, vsc = 1.f;
    if constexpr (FP8) {
        sl2 *= *p.k_scale;
        vsc = *p.v_scale;
    }
    const int32_t* bt_row = p.bt ? p.bt + (int64_t)r * p.bt_stride : nullptr;
    const int64_t rstride = (int64_t)p.Hkv * HD;
    const int64_t hoff = (int64_t)kh * HD;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* vl = smem + w * TILE * VP;

    for (int t0 = k_begin + w * TILE; t0 < k_end; t0 += NW * TILE) {
        // Each lane translates one key of the tile (lanes 32..63 repeat 0..31);
        // the row indices are then shared with the lanes that load that key.
        const int my_row = kv_row(bt_row, min(t0 + (lane & 31), L - 1), p.bs, q0);
        u32x4 kf[2][KS];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int rb = __shfl(my_row, b * 16 + row);
            const int64_t e0 = (int64_t)rb * rstride + hoff + G * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[b][ks] = load_kv8<FP8>(p.k_cache, e0 + ks * 32);
        }
        u32x4 vv[VLOADS];
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int c = lane + 64 * i;
            const int rv = __shfl(my_row, c / CPR);
            vv[i] = load_kv8<FP8>(p.v_cache, (int64_t)rv * rstride + hoff + (c % CPR) * 8);
        }
        // S^T[key][row] for two 16-key blocks
        f32x4 sacc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[b] = mfma16x16x32(kf[b][ks], qf[ks], sacc[b]);
        }
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kp = t0 + b * 16 + G * 4 + i;
                const float x = kp < limit ? sacc[b][i] * sl2 : -INFINITY;
                sv[b * 4 + i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sv[j] = fast_exp2(sv[j] - m_use);
            ps += sv[j];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < MB; ++i) oacc[i] *= alpha;
        // P^T as the B operand: k-slot 8*G + j holds key 16*(j/4) + 4*G + j%4
        const u32x4 pf = {pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]), pack_bf16x2(sv[4], sv[5]),
                          pack_bf16x2(sv[6], sv[7])};
        // V tile -> LDS (row-major), then V^T fragments by transposed reads
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int c = lane + 64 * i;
            *(u32x4*)(vl + (c / CPR) * VP + (c % CPR) * 8) = vv[i];
        }
        wave_lds_sync();
        const uint16_t* vt = vl + (G * 4 + ((lane & 15) >> 2)) * VP + (lane & 3) * 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const u32x2 lo = lds_read_tr16(vt + mb * 16);
            const u32x2 hi = lds_read_tr16(vt + 16 * VP + mb * 16);
            oacc[mb] = mfma16x16x32(u32x4{lo.x, lo.y, hi.x, hi.y}, pf, oacc[mb]);
        }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // merge the four waves' states
    __syncthreads();
    float* co = (float*)smem;  // [NW][16][HD]
    if (lane < 16) {
        sm_m[w][lane] = m_run;
        sm_l[w][lane] = l_run;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *(f32x4*)(co + (w * 16 + row) * HD + mb * 16 + G * 4) = oacc[mb];
    __syncthreads();

    constexpr int PER = HD / 16;
    const int frow = threadIdx.x >> 4;
    const int fc = (threadIdx.x & 15) * PER;
    if (frow >= rows_total) return;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i][frow]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float wt[NW], Lt = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        wt[i] = fast_exp2(sm_m[i][frow] - Mu);
        Lt += wt[i] * sm_l[i][frow];
    }
    const float inv = Lt > 0.f ? vsc / Lt : 0.f;
    float o[PER];
#pragma unroll
    for (int d = 0; d < PER; ++d) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) a += wt[i] * co[(i * 16 + frow) * HD + fc + d];
        o[d] = a * inv;
    }
    const float lse = Lt > 0.f ? (Mu + fast_log2(Lt)) * kLn2 : -INFINITY;
    const int64_t tok = q0 + frow / g;
    const int head = kh * g + frow % g;
    if (p.num_splits == 1) {
        store_bf16<PER>((uint16_t*)p.out + (tok * p.H + head) * HD + fc, o);
        if (p.lse && (threadIdx.x & 15) == 0) p.lse[(int64_t)head * p.T + tok] = lse;
    } else {
        store_f32<PER>(p.part_o + (((int64_t)s * p.T + tok) * p.H + head) * HD + fc, o);
        if ((threadIdx.x & 15) == 0) p.part_lse[((int64_t)s * p.H + head) * p.T + tok] = lse;
    }
}

// ----------------------------------------------------------------- prefill

template <int HD, bool FP8>
__global__ __launch_bounds__(256) void prefill_kernel(FwdParams p) {
    constexpr int TILE = kPrefillTile;
    constexpr int KP = HD + 8;          // LDS pitch of K rows (bf16 elements)
    constexpr int VP = HD + 16;         // LDS pitch of V rows
    constexpr int CPR = HD / 8;
    constexpr int LPT = TILE * CPR / 256;  // 16-byte chunks of K (and of V) per thread per tile
    constexpr int KS = HD / 16;         // k-steps of S^T = K Q^T (32x32x16)
    constexpr int MB = HD / 32;         // 32-row blocks of O^T
    static_assert(HD % 32 == 0 && LPT >= 1, "");
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[TILE * KP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[TILE * VP];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int nrk = p.B * p.Hkv;
    // longest-first: the highest query tiles (most keys under the causal mask) get the lowest ids
    const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / nrk);
    const int rk = blockIdx.x % nrk;
    const int r = rk / p.Hkv, kh = rk % p.Hkv;
    const int s = blockIdx.y;
    const int g = p.g;
    const int q0 = p.qsl[r];
    const int q_len = p.qsl[r + 1] - q0;
    const int tpw = kPrefillRows / g;   // tokens per work item
    const int tok0 = qt * tpw;
    if (tok0 >= q_len) return;
    const int L = p.seq_lens ? p.seq_lens[r] : q_len;
    const int ctx = L - q_len;
    const int tok_last = min(q_len, tok0 + tpw) - 1;
    const int item_end = p.causal ? min(L, ctx + tok_last + 1) : L;
    const int k_begin = p.num_splits > 1 ? s * p.split_len : 0;
    const int k_end = p.num_splits > 1 ? min(item_end, k_begin + p.split_len) : item_end;
    if (k_begin >= k_end) return;

    // this lane's query row
    const int rho = w * kPrefillRowsPerWave + (lane & 31);
    const int tl = tok0 + rho / g;
    const bool row_ok = rho < tpw * g && tl < q_len;
    const int head = kh * g + rho % g;
    int limit = p.causal ? min(L, ctx + tl + 1) : L;
    limit = row_ok ? min(limit, k_end) : 0;
    // the wave's key range: [k_begin, wave_max) holds every visible key of its rows;
    // keys below wave_min are visible to all of them
    const int wtok_first = tok0 + (w * kPrefillRowsPerWave) / g;
    const int wtok_last = min(min(q_len, tok0 + tpw) - 1, tok0 + (w * kPrefillRowsPerWave + 31) / g);
    const bool wave_any = wtok_first <= wtok_last && w * kPrefillRowsPerWave < tpw * g;
    const int wave_max = !wave_any ? k_begin : (p.causal ? min(k_end, ctx + wtok_last + 1) : k_end);
    const int wave_min = !wave_any ? k_begin : (p.causal ? min(k_end, ctx + wtok_first + 1) : k_end);

    u32x4 qf[KS];
    {
        const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(q0 + (row_ok ? tl : 0)) * p.H + head) * HD +
                             (lane >> 5) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? *(const u32x4*)(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    float sl2 = p.scale_log2, vsc = 1.f;
    if constexpr (FP8) {
        sl2 *= *p.k_scale;
        vsc = *p.v_scale;
    }
    const int32_t* bt_row = p.bt ? p.bt + (int64_t)r * p.bt_stride : nullptr;
    const int64_t rstride = (int64_t)p.Hkv * HD;
    const int64_t hoff = (int64_t)kh * HD;

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;

    // cooperative tile loads: thread -> chunks tid + 256*i
    u32x4 kreg[LPT], vreg[LPT];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = threadIdx.x + 256 * i;
            const int key = c / CPR;
            const int rw = kv_row(bt_row, min(t0 + key, L - 1), p.bs, q0);
            const int64_t e = (int64_t)rw * rstride + hoff + (c % CPR) * 8;
            kreg[i] = load_kv8<FP8>(p.k_cache, e);
            vreg[i] = load_kv8<FP8>(p.v_cache, e);
        }
    };
    load_tile(k_begin);
    const int hsel = lane >> 5;  // which half of the 32-row MFMA tile's k dimension this lane feeds
    for (int t0 = k_begin; t0 < k_end; t0 += TILE) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = threadIdx.x + 256 * i;
            *(u32x4*)(k_lds + (c / CPR) * KP + (c % CPR) * 8) = kreg[i];
            *(u32x4*)(v_lds + (c / CPR) * VP + (c % CPR) * 8) = vreg[i];
        }
        __syncthreads();
        if (t0 + TILE < k_end) load_tile(t0 + TILE);
        if (t0 >= wave_max) continue;  // tile entirely in this wave's future: skipped

        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
        const uint16_t* kr = k_lds + (lane & 31) * KP + hsel * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32x32x16(*(const u32x4*)(kr + ks * 16), qf[ks], sacc);

        const bool full = t0 + TILE <= wave_min;  // no element of this tile is masked for the wave
        float sv[16];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float x = sacc[e] * sl2;
            if (!full) {
                const int kp = t0 + (e >> 2) * 8 + hsel * 4 + (e & 3);
                x = kp < limit ? x : -INFINITY;
            }
            sv[e] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            sv[e] = fast_exp2(sv[e] - m_use);
            ps += sv[e];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < MB; ++i) oacc[i] *= alpha;
        u32x4 pf[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
            pf[k2] = u32x4{pack_bf16x2(sv[8 * k2 + 0], sv[8 * k2 + 1]), pack_bf16x2(sv[8 * k2 + 2], sv[8 * k2 + 3]),
                           pack_bf16x2(sv[8 * k2 + 4], sv[8 * k2 + 5]), pack_bf16x2(sv[8 * k2 + 6], sv[8 * k2 + 7])};
        // V^T fragments: lane group (hsel, c) reads keys 16*k2 + 8*jj + 4*hsel + e, columns 16*c + i
        const int grp_c = (lane >> 4) & 1;
        const uint16_t* vt = v_lds + (hsel * 4 + ((lane & 15) >> 2)) * VP + grp_c * 16 + (lane & 3) * 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const u32x2 lo = lds_read_tr16(vt + (16 * k2) * VP + mb * 32);
                const u32x2 hi = lds_read_tr16(vt + (16 * k2 + 8) * VP + mb * 32);
                oacc[mb] = mfma32x32x16(u32x4{lo.x, lo.y, hi.x, hi.y}, pf[k2], oacc[mb]);
            }
    }
    if (!row_ok) return;
    l_run += __shfl_xor(l_run, 32);
    const float inv = l_run > 0.f ? vsc / l_run : 0.f;
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    const float lse = l_run > 0.f ? (m_use + fast_log2(l_run)) * kLn2 : -INFINITY;
    const int64_t tok = q0 + tl;
    if (p.num_splits == 1) {
        uint16_t* op = (uint16_t*)p.out + (tok * p.H + head) * HD + hsel * 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float v4[4] = {oacc[mb][4 * q4] * inv, oacc[mb][4 * q4 + 1] * inv, oacc[mb][4 * q4 + 2] * inv,
                               oacc[mb][4 * q4 + 3] * inv};
                store_bf16<4>(op + mb * 32 + q4 * 8, v4);
            }
        if (p.lse && hsel == 0) p.lse[(int64_t)head * p.T + tok] = lse;
    } else {
        float* op = p.part_o + (((int64_t)s * p.T + tok) * p.H + head) * HD + hsel * 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(f32x4*)(op + mb * 32 + q4 * 8) =
                    f32x4{oacc[mb][4 * q4] * inv, oacc[mb][4 * q4 + 1] * inv, oacc[mb][4 * q4 + 2] * inv,
                          oacc[mb][4 * q4 + 3] * inv};
        if (hsel == 0) p.part_lse[((int64_t)s * p.H + head) * p.T + tok] = lse;
    }
}

// ----------------------------------------------------------------- generic

__device__ __forceinline__ int request_of(const int32_t* qsl, int B, int64_t tok) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <KvType KV>
__device__ __forceinline__ float load_kv1(const void* base, int64_t e) {
    if constexpr (KV == KvType::F32) return ((const float*)base)[e];
    else if constexpr (KV == KvType::BF16) return __uint_as_float((uint32_t)((const uint16_t*)base)[e] << 16);
    else return __builtin_amdgcn_cvt_f32_fp8((int)((const uint8_t*)base)[e], 0);
}

template <bool QF32, KvType KV>
__global__ __launch_bounds__(64) void generic_kernel(FwdParams p) {
    const int lane = threadIdx.x;
    const int64_t tok = blockIdx.x;
    const int h = blockIdx.y, s = blockIdx.z;
    const int r = request_of(p.qsl, p.B, tok);
    const int q0 = p.qsl[r];
    const int q_len = p.qsl[r + 1] - q0;
    const int t = (int)(tok - q0);
    const int L = p.seq_lens ? p.seq_lens[r] : q_len;
    const int n_vis = p.causal ? max(0, min(L, L - q_len + t + 1)) : L;
    const int k_begin = p.num_splits > 1 ? s * p.split_len : 0;
    const int k_end = p.num_splits > 1 ? min(n_vis, k_begin + p.split_len) : n_vis;
    if (p.num_splits > 1 && k_begin >= n_vis) return;
    const int hd = p.hd;
    const int kh = h / p.g;
    float qv[4], acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        const int64_t e = (tok * p.H + h) * hd + d;
        float x = 0.f;
        if (d < hd) x = QF32 ? ((const float*)p.q)[e] : __uint_as_float((uint32_t)((const uint16_t*)p.q)[e] << 16);
        qv[i] = x;
        acc[i] = 0.f;
    }
    float sl2 = p.scale_log2, vsc = 1.f;
    if constexpr (KV == KvType::FP8) {
        sl2 *= *p.k_scale;
        vsc = *p.v_scale;
    }
    const int32_t* bt_row = p.bt ? p.bt + (int64_t)r * p.bt_stride : nullptr;
    const int64_t rstride = (int64_t)p.Hkv * hd;
    float m = -INFINITY, l = 0.f;
    for (int j = k_begin; j < k_end; ++j) {
        const int64_t base = (int64_t)kv_row(bt_row, j, p.bs, q0) * rstride + (int64_t)kh * hd;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = lane + 64 * i;
            if (d < hd) dot += qv[i] * load_kv1<KV>(p.k_cache, base + d);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
        const float x = dot * sl2;
        const float m_new = fmaxf(m, x);
        const float alpha = fast_exp2(m - m_new);
        const float pj = fast_exp2(x - m_new);
        l = l * alpha + pj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = lane + 64 * i;
            acc[i] = acc[i] * alpha + (d < hd ? pj * load_kv1<KV>(p.v_cache, base + d) : 0.f);
        }
        m = m_new;
    }
    const float inv = l > 0.f ? vsc / l : 0.f;
    const float lse = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d >= hd) continue;
        const float o = acc[i] * inv;
        if (p.num_splits == 1) {
            const int64_t e = (tok * p.H + h) * hd + d;
            if (QF32) ((float*)p.out)[e] = o;
            else ((uint16_t*)p.out)[e] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xFFFFu);
        } else {
            p.part_o[(((int64_t)s * p.T + tok) * p.H + h) * hd + d] = o;
        }
    }
    if (lane == 0) {
        if (p.num_splits == 1) {
            if (p.lse) p.lse[(int64_t)h * p.T + tok] = lse;
        } else {
            p.part_lse[((int64_t)s * p.H + h) * p.T + tok] = lse;
        }
    }
}

// ----------------------------------------------------------------- combine

// One thread per 4 output elements. Split s of a row holds keys
// [s * split_len, (s+1) * split_len); only splits below ceil(n_vis / split_len)
// were written, and only those are read.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cpr = p.hd / 4;
    const int64_t nrow = p.T * p.H;
    if (idx >= nrow * cpr) return;
    const int64_t rowi = idx / cpr;
    const int c = (int)(idx % cpr);
    const int64_t tok = rowi / p.H;
    const int h = (int)(rowi % p.H);
    const int r = request_of(p.qsl, p.B, tok);
    const int q0 = p.qsl[r];
    const int q_len = p.qsl[r + 1] - q0;
    const int L = p.seq_lens ? p.seq_lens[r] : q_len;
    const int t = (int)(tok - q0);
    const int n_vis = p.causal ? max(0, min(L, L - q_len + t + 1)) : L;
    const int n_valid = min(p.num_splits, (n_vis + p.split_len - 1) / p.split_len);
    float M = -INFINITY;
    for (int s = 0; s < n_valid; ++s) M = fmaxf(M, p.part_lse[((int64_t)s * p.H + h) * p.T + tok]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (M != -INFINITY) {
        float sum = 0.f;
        for (int s = 0; s < n_valid; ++s) {
            const float ls = p.part_lse[((int64_t)s * p.H + h) * p.T + tok];
            const float wgt = fast_exp2((ls - M) * kLog2e);
            sum += wgt;
            const f32x4 v = *(const f32x4*)(p.part_o + (((int64_t)s * p.T + tok) * p.H + h) * p.hd + 4 * c);
            o += wgt * v;
        }
        o *= 1.f / sum;
        lse = M + fast_log2(sum) * kLn2;
    }
    const int64_t e = (tok * p.H + h) * p.hd + 4 * c;
    if (OUT_F32) {
        *(f32x4*)((float*)p.out + e) = o;
    } else {
        *(u32x2*)((uint16_t*)p.out + e) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    if (p.lse && c == 0) p.lse[(int64_t)h * p.T + tok] = lse;
}

template <bool F32>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t e) {
    if constexpr (F32) {
        return *(const f32x4*)((const float*)base + e);
    } else {
        const u32x2 w = *(const u32x2*)((const uint16_t*)base + e);
        return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    }
}

template <bool F32>
__global__ __launch_bounds__(256) void merge_kernel(void* out, float* out_lse, const void* po, const float* plse,
                                                    const void* so, const float* slse, int64_t T, int H, int hd) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cpr = hd / 4;
    if (idx >= T * H * cpr) return;
    const int64_t rowi = idx / cpr;
    const int c = (int)(idx % cpr);
    const int64_t tok = rowi / H;
    const int h = (int)(rowi % H);
    const float a = plse[(int64_t)h * T + tok], b = slse[(int64_t)h * T + tok];
    const float M = fmaxf(a, b);
    const int64_t e = rowi * hd + 4 * c;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (M != -INFINITY) {
        const float wa = fast_exp2((a - M) * kLog2e), wb = fast_exp2((b - M) * kLog2e);
        const float inv = 1.f / (wa + wb);
        o = (wa * inv) * load4<F32>(po, e) + (wb * inv) * load4<F32>(so, e);
        lse = M + fast_log2(wa + wb) * kLn2;
    }
    if (F32) {
        *(f32x4*)((float*)out + e) = o;
    } else {
        *(u32x2*)((uint16_t*)out + e) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    if (out_lse && c == 0) out_lse[(int64_t)h * T + tok] = lse;
}

// ----------------------------------------------------------------- launchers

template <int HD>
static hipError_t decode_hd(const FwdParams& p, KvType kv, hipStream_t s) {
    dim3 grid(p.num_splits, p.Hkv, p.B);
    if (kv == KvType::FP8) hipLaunchKernelGGL((decode_kernel<HD, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<HD, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_decode(const FwdParams& p, KvType kv, hipStream_t s) {
    switch (p.hd) {
        case 64: return decode_hd<64>(p, kv, s);
        case 128: return decode_hd<128>(p, kv, s);
        case 256: return decode_hd<256>(p, kv, s);
        default: return hipErrorInvalidValue;
    }
}

template <int HD>
static hipError_t prefill_hd(const FwdParams& p, KvType kv, hipStream_t s) {
    dim3 grid((unsigned)p.n_qtiles * p.B * p.Hkv, p.num_splits);
    if (kv == KvType::FP8) hipLaunchKernelGGL((prefill_kernel<HD, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prefill_kernel<HD, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_prefill(const FwdParams& p, KvType kv, hipStream_t s) {
    switch (p.hd) {
        case 64: return prefill_hd<64>(p, kv, s);
        case 128: return prefill_hd<128>(p, kv, s);
        case 256: return prefill_hd<256>(p, kv, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_generic(const FwdParams& p, KvType kv, bool q_f32, hipStream_t s) {
    dim3 grid((unsigned)p.T, p.H, p.num_splits);
    if (q_f32) hipLaunchKernelGGL((generic_kernel<true, KvType::F32>), grid, dim3(64), 0, s, p);
    else if (kv == KvType::FP8) hipLaunchKernelGGL((generic_kernel<false, KvType::FP8>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((generic_kernel<false, KvType::BF16>), grid, dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_combine(const FwdParams& p, bool out_f32, hipStream_t s) {
    const int64_t n = p.T * p.H * (p.hd / 4);
    dim3 grid((unsigned)((n + 255) / 256));
    if (out_f32) hipLaunchKernelGGL((combine_kernel<true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_merge(void* out, float* out_lse, const void* po, const float* plse, const void* so,
                        const float* slse, int64_t T, int32_t H, int32_t hd, bool f32, hipStream_t s) {
    const int64_t n = T * H * (hd / 4);
    dim3 grid((unsigned)((n + 255) / 256));
    if (f32) hipLaunchKernelGGL((merge_kernel<true>), grid, dim3(256), 0, s, out, out_lse, po, plse, so, slse, T, H, hd);
    else hipLaunchKernelGGL((merge_kernel<false>), grid, dim3(256), 0, s, out, out_lse, po, plse, so, slse, T, H, hd);
    return hipGetLastError();
}

}  // namespace pkv
