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
//  decode_balanced_kernel
//                  the 32-key tiles of every (request, kv head) item laid end
//                  to end and dealt out in equal contiguous shares to a grid of
//                  waves that is resident at once; items of up to 32 query rows
//                  as one or two 16-column blocks of the 16x16x32 MFMA, tiles
//                  copied straight into LDS (two stages per wave), one partial
//                  state per item segment a wave covers (a whole item: the
//                  final output).
//  prefill_kernel  one work item = (request, kv head, 128 query rows, KV split);
//                  rows are (token, head-of-group) pairs, 32 per wave, on the
//                  32x32x16 bf16 MFMA (32x32x64 fp8 for Q K^T with an fp8 q);
//                  64-key K/V tiles are copied from HBM straight into padded
//                  row-major LDS (16-byte chunks permuted per row; two slots
//                  each, one tile ahead) and shared by the four waves; only
//                  tiles crossing the diagonal build a per-element mask. Items
//                  of at most 64 rows run key-split: two waves per 32 rows, each
//                  on one 32-key half of every tile, folded at the end.
//  generic_kernel  one wave per (token, head); plain fp32 arithmetic on the
//                  vector ALUs for fp32 inputs and head sizes without an MFMA
//                  instantiation.
//  combine_kernel  log-sum-exp merge of the KV-split partials of the above.
//  combine_balanced_kernel
//                  log-sum-exp merge of the balanced decode's partial states.
//  combine_cascade_kernel
//                  the same for a cascade run as one balanced decode: each
//                  suffix row folded with the shared-prefix item's row.
//  merge_kernel    merge of two attention states (cascade prefix / suffix).
#include <type_traits>

#include "pkv_common.h"

namespace pkv {

// ----------------------------------------------------------------- decode

// One decode wave's 32-key tile: loads, LDS staging and compute. The LDS area
// of a wave holds the tile's K and V row-major in bf16. The K pitch (HD + 8
// elements) puts consecutive rows 16 bytes apart in bank space, so the
// 16-byte A-operand reads of 8 consecutive rows hit 32 distinct banks; the V
// pitch (HD + 16) does the same for the transposed 8-byte reads.
template <int HD, bool FP8>
struct DecodeTile {
    static constexpr int TILE = kDecodeTile;
    static constexpr int KS = HD / 32;         // k-steps of S^T = K Q^T
    static constexpr int MB = HD / 16;         // 16-row blocks of O^T
    static constexpr int KP = HD + 8;
    static constexpr int VP = HD + 16;
    static constexpr int K_ELEMS = TILE * KP;
    static constexpr int ELEMS = TILE * (KP + VP);  // bf16 elements per wave
    static constexpr int ESZ = FP8 ? 1 : 2;    // bytes per cached element
    static constexpr int EPL = 16 / ESZ;       // elements per 16-byte load
    static constexpr int GPR = HD / EPL;       // 16-byte loads per cache row (one kv head)
    static constexpr int NL = TILE * GPR / 64; // loads per lane per tile, for K and again for V
    static_assert(HD % 32 == 0 && 64 % GPR == 0 && NL >= 1, "");

    static constexpr int KPL = 64 / GPR;       // keys per load instruction

    // Key (within the tile) that load i of `lane` reads.
    static __device__ __forceinline__ int key_of(int lane, int i) { return lane / GPR + KPL * i; }

    // Tiles of head size 128 can go straight from the cache into LDS
    // (global_load_lds, no registers on the way), into two stages per wave so
    // that the next tile lands while this one is computed. A K or V tile is
    // then 32 rows of 256 bytes (bf16) or 128 bytes (fp8, kept as bytes and
    // widened as it is read), row r at its row offset with its 16-byte chunk
    // c at position c ^ dsw(r) (each copy lane fetches the chunk its position
    // needs). dsw permutes row bits so that the rows of a K operand read and
    // of 32 lanes' transposed V reads hit every one of the 64 banks once.
    static constexpr bool DMA = HD == 128;
    static constexpr int ROW_BYTES = HD * ESZ;                // bytes of a row
    static constexpr int DMA_TILE = TILE * ROW_BYTES;         // bytes of a K or V tile
    static constexpr int DMA_STAGE = 2 * DMA_TILE;      // K then V
    static __device__ __forceinline__ int dsw(int r) {
        if constexpr (FP8)  // 8 chunks a row: the even (odd) rows of a read take 8 distinct positions
            return ((r >> 1) & 3) | ((((r >> 3) ^ (r >> 4)) & 1) << 2);
        else
            return (((r >> 2) & 1) << 3) | (((r >> 1) & 1) << 2) | ((r & 1) << 1) | ((r >> 3) & 1);
    }
    static __device__ __forceinline__ void issue(const FwdParams& p, int lane, const int (&rows)[NL], int kh,
                                                 uint8_t* st) {
        const int64_t rstride = (int64_t)p.Hkv * HD;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int chunk = (lane % GPR) ^ dsw(key_of(lane, i));
            const int64_t e = ((int64_t)rows[i] * rstride + (int64_t)kh * HD + chunk * EPL) * ESZ;
            copy16_to_lds<0>((const uint8_t*)p.k_cache + e, st + i * 1024);
            copy16_to_lds<0>((const uint8_t*)p.v_cache + e, st + DMA_TILE + i * 1024);
        }
    }

    // K and V of a tile with row-coalesced 16-byte loads: load i of lane l
    // covers granule c = l + 64 i, i.e. key c / GPR, elements (c % GPR) * EPL
    // onward, so each group of GPR consecutive lanes reads one whole cache row
    // of the kv head. (Reading K in the MFMA operand layout instead, 16 keys x
    // 64 bytes per instruction, streams far below the HBM rate.) rows[i] is
    // the cache row of key key_of(lane, i); every lane translates its own
    // keys, so issuing the loads needs no cross-lane traffic.
    static __device__ __forceinline__ void load(const FwdParams& p, int lane, const int (&rows)[NL], int kh,
                                                u32x4 (&kr)[NL], u32x4 (&vr)[NL]) {
        const int64_t rstride = (int64_t)p.Hkv * HD;
        const int64_t col = (int64_t)kh * HD + (lane % GPR) * EPL;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int64_t e = (int64_t)rows[i] * rstride + col;
            kr[i] = *(const u32x4*)((const uint8_t*)p.k_cache + e * ESZ);
            vr[i] = *(const u32x4*)((const uint8_t*)p.v_cache + e * ESZ);
        }
    }
    // registers -> LDS, row-major bf16 (fp8 widened, exactly)
    static __device__ __forceinline__ void store(uint16_t* stage, int lane, const u32x4 (&kr)[NL],
                                                 const u32x4 (&vr)[NL]) {
        uint16_t* const kl = stage;
        uint16_t* const vl = stage + K_ELEMS;
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int c = lane + 64 * i;
            const int key = c / GPR, col = (c % GPR) * EPL;
            if constexpr (FP8) {
                *(u32x4*)(kl + key * KP + col) = fp8x8_to_bf16x8(u32x2{kr[i].x, kr[i].y});
                *(u32x4*)(kl + key * KP + col + 8) = fp8x8_to_bf16x8(u32x2{kr[i].z, kr[i].w});
                *(u32x4*)(vl + key * VP + col) = fp8x8_to_bf16x8(u32x2{vr[i].x, vr[i].y});
                *(u32x4*)(vl + key * VP + col + 8) = fp8x8_to_bf16x8(u32x2{vr[i].z, vr[i].w});
            } else {
                *(u32x4*)(kl + key * KP + col) = kr[i];
                *(u32x4*)(vl + key * VP + col) = vr[i];
            }
        }
        wave_lds_sync();
    }
    // One tile from LDS: S^T with K as the A operand and the item's query
    // rows as the 16 columns, masking keys at or past `limit` (per row) and,
    // with the variants compiled in (VAR), keys before `lo`, applying the
    // soft cap (cap_l2 > 0) and the ALiBi bias (slope al2, query position
    // qpos),
    // online softmax, then O^T += V^T P^T with V^T read transposed. m_run is
    // row-uniform (log2 domain), l_run per lane (this lane's keys only), and
    // lc_run the same sum over the probabilities as rounded to bf16 for PV.
    // (DL: the tile is in the global_load_lds layout above)
    template <bool VAR, bool DL = false>
    static __device__ __forceinline__ void compute(const uint16_t* stage, int lane, int t0, int lo, int limit,
                                                   float sl2, float cap_l2, float cap_inv2, float al2, int qpos,
                                                   const u32x4 (&qf)[KS], float& m_run, float& l_run,
                                                   float& lc_run, f32x4 (&oacc)[MB]) {
        const uint16_t* const kl = stage;
        const uint16_t* const vl = stage + K_ELEMS;
        const uint8_t* const st = (const uint8_t*)stage;
        const int row = lane & 15;
        const int G = lane >> 4;
        f32x4 sacc[2];
        const uint16_t* kp = kl + row * KP + G * 8;
        // DL, bf16: row b 16 + row, chunk G + 4 ks at position (G + 4 ks) ^ dsw(row);
        // fp8: bytes 32 ks + 8 G of the row, chunk 2 ks + G / 2, half G % 2
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int swk = dsw(b * 16 + row);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 kf;
                if constexpr (DL && FP8)
                    kf = fp8x8_to_bf16x8(*(const u32x2*)(st + (b * 16 + row) * ROW_BYTES +
                                                         (((2 * ks + (G >> 1)) ^ swk) << 4) + (G & 1) * 8));
                else if constexpr (DL)
                    kf = *(const u32x4*)(st + (b * 16 + row) * ROW_BYTES + (((G + 4 * ks) ^ swk) << 4));
                else
                    kf = *(const u32x4*)(kp + b * 16 * KP + ks * 32);
                sacc[b] = mfma16x16x32(kf, qf[ks], sacc[b]);
            }
        }
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = t0 + b * 16 + G * 4 + i;
                float x = sacc[b][i] * sl2;
                if constexpr (VAR) {
                    if (cap_l2 > 0.f) x = softcap_l2(x, cap_l2, cap_inv2);
                    if (al2 != 0.f) x -= al2 * fabsf((float)(qpos - key));
                    x = key < limit && key >= lo ? x : -INFINITY;
                } else {
                    x = key < limit ? x : -INFINITY;
                }
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
        lc_run = add_bf16_pair(pf.w, add_bf16_pair(pf.z, add_bf16_pair(pf.y, add_bf16_pair(pf.x, lc_run * alpha))));
        const uint16_t* vt = vl + (G * 4 + ((lane & 15) >> 2)) * VP + (lane & 3) * 4;
        // DL, bf16: row R (and R + 16), bytes 32 mb + 8 (lane & 3) onward:
        // chunk 2 mb + (lane & 3) / 2 at position chunk ^ dsw(R), half lane & 1.
        // fp8: one transposed byte read gives the 8 keys of the lane's k-slots;
        // lane s of a 16-lane group addresses bytes 16 mb + 8 (s % 2) of the
        // row of slot s / 2 (key 16 (j / 4) + 4 G + j % 4, j = s / 2).
        const int rv = FP8 ? 16 * (((lane & 15) >> 1) >> 2) + 4 * G + (((lane & 15) >> 1) & 3)
                           : G * 4 + ((lane & 15) >> 2);
        const int swv = dsw(rv);
        const uint8_t* const vst = st + DMA_TILE + rv * ROW_BYTES + (lane & 1) * 8;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            u32x4 vf;
            if constexpr (DL && FP8) {
                vf = fp8x8_to_bf16x8(lds_read_tr8(vst + ((mb ^ swv) << 4)));
            } else {
                u32x2 lo, hi;
                if constexpr (DL) {
                    const int pos = ((2 * mb + ((lane & 3) >> 1)) ^ swv) << 4;
                    lo = lds_read_tr16(vst + pos);
                    hi = lds_read_tr16(vst + 16 * ROW_BYTES + pos);
                } else {
                    lo = lds_read_tr16(vt + mb * 16);
                    hi = lds_read_tr16(vt + 16 * VP + mb * 16);
                }
                vf = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
            oacc[mb] = mfma16x16x32(vf, pf, oacc[mb]);
        }
    }

    // The first N of an item's RB blocks of 16 query rows over one tile, as
    // compute() does for one block, except that every K and V fragment read
    // from LDS feeds the MFMAs of all N blocks, and that the running output is
    // rescaled lazily: only when some row's tile maximum exceeds its running
    // maximum by more than kLazyRescale (log2 domain; a wave-uniform
    // decision), so that the probabilities stay below 2^kLazyRescale and the
    // accumulators are otherwise touched by the MFMAs alone.
    template <bool VAR, bool DL, int N, int RB>
    static __device__ __forceinline__ void compute_rows(const uint16_t* stage, int lane, int t0, const int (&lo)[RB],
                                                        const int (&limit)[RB], float sl2, float cap_l2,
                                                        float cap_inv2, const float (&al2)[RB], const int (&qpos)[RB],
                                                        const u32x4 (&qf)[RB][KS], float (&m_run)[RB],
                                                        float (&l_run)[RB], float (&lc_run)[RB],
                                                        f32x4 (&oacc)[RB][MB]) {
        static_assert(N >= 1 && N <= RB, "");
        const uint16_t* const kl = stage;
        const uint16_t* const vl = stage + K_ELEMS;
        const uint8_t* const st = (const uint8_t*)stage;
        const int row = lane & 15;
        const int G = lane >> 4;
        f32x4 sacc[N][2];
        const uint16_t* kp = kl + row * KP + G * 8;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int n = 0; n < N; ++n) sacc[n][b] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int swk = dsw(b * 16 + row);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 kf;
                if constexpr (DL && FP8)
                    kf = fp8x8_to_bf16x8(*(const u32x2*)(st + (b * 16 + row) * ROW_BYTES +
                                                         (((2 * ks + (G >> 1)) ^ swk) << 4) + (G & 1) * 8));
                else if constexpr (DL)
                    kf = *(const u32x4*)(st + (b * 16 + row) * ROW_BYTES + (((G + 4 * ks) ^ swk) << 4));
                else
                    kf = *(const u32x4*)(kp + b * 16 * KP + ks * 32);
#pragma unroll
                for (int n = 0; n < N; ++n) sacc[n][b] = mfma16x16x32(kf, qf[n][ks], sacc[n][b]);
            }
        }
        u32x4 pf[N];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float sv[8];
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = t0 + b * 16 + G * 4 + i;
                    float x = sacc[n][b][i] * sl2;
                    if constexpr (VAR) {
                        if (cap_l2 > 0.f) x = softcap_l2(x, cap_l2, cap_inv2);
                        if (al2[n] != 0.f) x -= al2[n] * fabsf((float)(qpos[n] - key));
                        x = key < limit[n] && key >= lo[n] ? x : -INFINITY;
                    } else {
                        x = key < limit[n] ? x : -INFINITY;
                    }
                    sv[b * 4 + i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (__any(mx > m_run[n] + kLazyRescale)) {
                const float m_new = fmaxf(m_run[n], mx);
                const float alpha = fast_exp2(m_run[n] - (m_new == -INFINITY ? 0.f : m_new));
                l_run[n] *= alpha;
                lc_run[n] *= alpha;
#pragma unroll
                for (int i = 0; i < MB; ++i) oacc[n][i] *= alpha;
                m_run[n] = m_new;
            }
            const float m_use = m_run[n] == -INFINITY ? 0.f : m_run[n];
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sv[j] = fast_exp2(sv[j] - m_use);
                ps += sv[j];
            }
            l_run[n] += ps;
            pf[n] = u32x4{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]), pack_bf16x2(sv[4], sv[5]),
                          pack_bf16x2(sv[6], sv[7])};
            lc_run[n] = add_bf16_pair(pf[n].w, add_bf16_pair(pf[n].z, add_bf16_pair(pf[n].y,
                                                                                 add_bf16_pair(pf[n].x, lc_run[n]))));
        }
        const uint16_t* vt = vl + (G * 4 + ((lane & 15) >> 2)) * VP + (lane & 3) * 4;
        const int rv = FP8 ? 16 * (((lane & 15) >> 1) >> 2) + 4 * G + (((lane & 15) >> 1) & 3)
                           : G * 4 + ((lane & 15) >> 2);
        const int swv = dsw(rv);
        const uint8_t* const vst = st + DMA_TILE + rv * ROW_BYTES + (lane & 1) * 8;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            u32x4 vf;
            if constexpr (DL && FP8) {
                vf = fp8x8_to_bf16x8(lds_read_tr8(vst + ((mb ^ swv) << 4)));
            } else {
                u32x2 lo2, hi2;
                if constexpr (DL) {
                    const int pos = ((2 * mb + ((lane & 3) >> 1)) ^ swv) << 4;
                    lo2 = lds_read_tr16(vst + pos);
                    hi2 = lds_read_tr16(vst + 16 * ROW_BYTES + pos);
                } else {
                    lo2 = lds_read_tr16(vt + mb * 16);
                    hi2 = lds_read_tr16(vt + 16 * VP + mb * 16);
                }
                vf = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
            }
#pragma unroll
            for (int n = 0; n < N; ++n) oacc[n][mb] = mfma16x16x32(vf, pf[n], oacc[n][mb]);
        }
    }
};

// Query fragment of a decode item: lane l feeds row row0 + l % 16 (token
// row / g, head kh * g + row % g), head-dim elements 8 * (l / 16) + 32 ks
// onward.
template <int HD>
__device__ __forceinline__ void load_decode_q(const FwdParams& p, int lane, int q0, int rows_total, int kh,
                                              u32x4 (&qf)[HD / 32], int row0 = 0) {
    const int row = row0 + (lane & 15);
    const bool row_ok = row < rows_total;
    const int tl = row_ok ? row / p.g : 0;
    const int hh = kh * p.g + (row_ok ? row % p.g : 0);
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(q0 + tl) * p.H + hh) * HD + (lane >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) qf[ks] = row_ok ? *(const u32x4*)(qp + ks * 32) : u32x4{0u, 0u, 0u, 0u};
}

// First key query row row0 + lane % 16 of an item may see (the sliding window).
__device__ __forceinline__ int decode_row_lo(const FwdParams& p, int lane, int q_len, int L, int row0 = 0) {
    const int row = row0 + (lane & 15);
    if (row >= q_len * p.g) return 0;
    return window_lo(p, L - q_len + row / p.g);
}

// Sequence position and log2-domain ALiBi slope of query row row0 + lane % 16.
__device__ __forceinline__ int decode_row_pos(const FwdParams& p, int lane, int q_len, int L, int row0 = 0) {
    return L - q_len + (row0 + (lane & 15)) / p.g;
}
__device__ __forceinline__ float decode_row_alibi(const FwdParams& p, int lane, int kh, int row0 = 0) {
    return alibi_l2(p, kh * p.g + (row0 + (lane & 15)) % p.g);
}

// Largest key index + 1 that query row row0 + lane % 16 of an item may see.
__device__ __forceinline__ int decode_row_limit(const FwdParams& p, int lane, int q_len, int L, bool causal,
                                                int row0 = 0) {
    const int row = row0 + (lane & 15);
    if (row >= q_len * p.g) return 0;
    return causal ? min(L, L - q_len + row / p.g + 1) : L;
}

// One wave's share of a decode work item: keys [k_first, k_end) of request r,
// kv head kh, taken in 32-key tiles k_first, k_first + step, ... (step is a
// multiple of 32). The item's query rows (q_len tokens x g heads of the group,
// at most 16) are the columns of 16x16x32 MFMAs: S^T = K Q^T, O^T += V^T P^T.
// `stage` is the wave's LDS area. Returns the wave's online-softmax state: m
// (log2 domain, row-uniform), l (summed over the row), and O^T (lane holds
// row l%16, head-dim elements 16*mb + 4*(l/16) + i).
template <int HD, bool FP8, bool PAGED, bool VAR>
__device__ __forceinline__ void decode_range(const FwdParams& p, uint16_t* stage, int lane, int r, int kh, int q0,
                                             int q_len, int L, int k_first, int step, int k_end, float& m_run,
                                             float& l_run, float& lc_run, f32x4 (&oacc)[HD / 16]) {
    using DT = DecodeTile<HD, FP8>;
    constexpr int NL = DT::NL;
    u32x4 qf[DT::KS];
    load_decode_q<HD>(p, lane, q0, q_len * p.g, kh, qf);
    const int limit = min(decode_row_limit(p, lane, q_len, L, p.causal), k_end);
    const int lo = VAR ? decode_row_lo(p, lane, q_len, L) : 0;
    const float al2 = VAR ? decode_row_alibi(p, lane, kh) : 0.f;
    const int qpos = decode_row_pos(p, lane, q_len, L);
    float sl2 = p.scale_log2;
    if constexpr (FP8) sl2 *= *p.k_scale;
    const int32_t* bt_row = PAGED ? p.bt + (int64_t)r * p.bt_stride : nullptr;

    m_run = -INFINITY;
    l_run = 0.f;
    lc_run = 0.f;
#pragma unroll
    for (int i = 0; i < DT::MB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Address translation is split in two so that the block-table loads of a
    // tile can be issued a full tile ahead of their use: page_for issues the
    // loads of the block-table entries of the keys this lane will read in
    // tile t, row_from turns them into cache rows when the tile's loads are
    // issued. (Using an entry right after loading it would make the wave wait
    // for every load in flight, since loads retire in order.) Keys at or past
    // the end of the range are clamped to its last key, so a prefetch past
    // the end re-reads one cached row and every address stays inside the
    // request's pages.
    auto page_for = [&](int t, int (&pg)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int pos = min(t + DT::key_of(lane, i), k_end - 1);
            if constexpr (PAGED) pg[i] = bt_row[page_index(pos, p.bs, p.bs_shift)];
            else pg[i] = q0 + pos;
        }
    };
    auto row_from = [&](int t, const int (&pg)[NL], int (&rows)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int pos = min(t + DT::key_of(lane, i), k_end - 1);
            if constexpr (PAGED) rows[i] = pg[i] * p.bs + page_offset(pos, p.bs, p.bs_shift);
            else rows[i] = pg[i];
        }
    };

    // Software pipeline over the wave's tiles. Iteration i: request the
    // block-table entries of tile i+2, issue the K/V loads of tile i+1
    // (unconditionally: past the end they re-read a cached row), compute tile
    // i from LDS, turn the block-table entries into row indices, and move tile
    // i+1 into LDS. Every load result is consumed in the iteration that
    // issued it, so the wait before the LDS stores covers that tile only.
    int t_cur = k_first;
    if (t_cur < k_end) {
        u32x4 kr[NL], vr[NL];
        int pg[NL], rows[NL];
        page_for(t_cur, pg);
        row_from(t_cur, pg, rows);
        page_for(t_cur + step, pg);
        DT::load(p, lane, rows, kh, kr, vr);
        row_from(t_cur + step, pg, rows);
        DT::store(stage, lane, kr, vr);
        while (true) {
            page_for(t_cur + 2 * step, pg);
            DT::load(p, lane, rows, kh, kr, vr);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch issued before the compute
            DT::template compute<VAR>(stage, lane, t_cur, lo, limit, sl2, p.softcap_l2, p.softcap_inv2, al2, qpos,
                                      qf, m_run, l_run, lc_run, oacc);
            row_from(t_cur + 2 * step, pg, rows);
            t_cur += step;
            if (t_cur >= k_end) break;
            DT::store(stage, lane, kr, vr);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // per-row sums over the four lane groups
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    lc_run += __shfl_xor(lc_run, 16);
    lc_run += __shfl_xor(lc_run, 32);
}

// Split-KV decode: one workgroup per (KV split, kv head, request); its four
// waves take interleaved tiles of the split and merge their states in LDS.
// VAR: the sliding window / soft cap code is compiled in (sinks cost
// nothing when absent and are always handled).
template <int HD, bool FP8, bool PAGED, bool VAR>
__global__ __launch_bounds__(256, HD <= 128 ? 2 : 1) void decode_kernel(FwdParams p) {
    constexpr int TILE = kDecodeTile;
    constexpr int NW = kDecodeWaves;
    constexpr int MB = HD / 16;
    constexpr int VSM = NW * DecodeTile<HD, FP8>::ELEMS;  // bf16 elements of K/V staging
    constexpr int OSM = NW * 16 * HD * 2;           // the same bytes reused as fp32 partial outputs
    __shared__ __attribute__((aligned(16))) uint16_t smem[VSM > OSM ? VSM : OSM];
    __shared__ float sm_m[NW][16], sm_l[NW][16], sm_lc[NW][16];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
    const int s = blockIdx.x, kh = blockIdx.y, r = blockIdx.z;
    const int q0 = req_q0(p, r);
    const int q_len = req_qend(p, r) - q0;
    if (q_len <= 0) return;
    const int L = req_L(p, r, q_len);
    const int base = VAR ? window_base(p, q_len, L) : 0;
    const int k_begin = base + (p.num_splits > 1 ? s * p.split_len : 0);
    const int k_end = p.num_splits > 1 ? min(L, k_begin + p.split_len) : L;
    if (k_begin >= k_end) return;  // no row of this item sees a key here; the merge never reads it

    float m_run, l_run, lc_run;
    f32x4 oacc[MB];
    decode_range<HD, FP8, PAGED, VAR>(p, smem + w * DecodeTile<HD, FP8>::ELEMS, lane, r, kh, q0, q_len, L, k_begin + w * TILE,
                                 NW * TILE,
                                 k_end, m_run, l_run, lc_run, oacc);
    const int row = lane & 15;
    const int G = lane >> 4;
    const int g = p.g;
    const int rows_total = q_len * g;

    // merge the four waves' states
    __syncthreads();
    float* co = (float*)smem;  // [NW][16][HD]
    if (lane < 16) {
        sm_m[w][lane] = m_run;
        sm_l[w][lane] = l_run;
        sm_lc[w][lane] = lc_run;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *(f32x4*)(co + (w * 16 + row) * HD + mb * 16 + G * 4) = oacc[mb];
    __syncthreads();

    constexpr int PER = HD / 16;
    const int frow = threadIdx.x >> 4;
    const int fc = (threadIdx.x & 15) * PER;
    if (frow >= rows_total) return;
    const float vsc = FP8 ? *p.v_scale : 1.f;
    const int64_t tok = q0 + frow / g;
    const int head = kh * g + frow % g;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i][frow]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float wt[NW], Lt = 0.f, Ltc = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        wt[i] = fast_exp2(sm_m[i][frow] - Mu);
        Lt += wt[i] * sm_l[i][frow];
        Ltc += wt[i] * sm_lc[i][frow];
    }
    // the sink joins the normaliser once, in the final output (split
    // partials leave it to the merge)
    float inv, lse;
    finalize_row(M, Lt, Ltc, p.num_splits == 1 ? sink_l2(p, head) : -INFINITY, vsc, inv, lse);
    float o[PER];
#pragma unroll
    for (int d = 0; d < PER; ++d) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) a += wt[i] * co[(i * 16 + frow) * HD + fc + d];
        o[d] = a * inv;
    }
    if (p.num_splits == 1) {
        store_bf16<PER>((uint16_t*)p.out + (tok * p.H + head) * HD + fc, o);
        if (p.lse && (threadIdx.x & 15) == 0) p.lse[(int64_t)head * p.T + tok] = lse;
    } else {
        store_f32<PER>(p.part_o + (((int64_t)s * p.T + tok) * p.H + head) * HD + fc, o);
        if ((threadIdx.x & 15) == 0) p.part_lse[((int64_t)s * p.H + head) * p.T + tok] = lse;
    }
}

// ------------------------------------------------- decode, balanced schedule
//
// Every (request, kv head) item of decode is a row of 32-key tiles; the items
// are laid end to end (request-major, then kv head) into one list of N tiles
// and wave w of the grid takes tiles [w N / W, (w+1) N / W), whatever items
// they belong to. Each wave therefore streams the same number of bytes, and
// the grid is sized to be resident at once. A wave writes one partial state
// per item segment it covers, into slot (w + item); when it covers a whole
// item it writes the final output instead. The merge kernel then combines,
// for each row, the partials of the waves wave_of(first tile of its item) ..
// wave_of(last tile), which are exactly the waves that wrote them.

// Tiles of one item of request r: from the window base (0 without a
// window) to the last key.
// (VAR false: no window, known at compile time.)
template <bool VAR = true>
__device__ __forceinline__ int decode_first_tile(const FwdParams& p, int q_len, int L) {
    return VAR ? window_base(p, q_len, L) / kDecodeTile : 0;
}
template <bool VAR = true>
__device__ __forceinline__ int decode_tiles_of(const FwdParams& p, int q_len, int L) {
    return q_len <= 0 ? 0 : (L + kDecodeTile - 1) / kDecodeTile - decode_first_tile<VAR>(p, q_len, L);
}
template <bool VAR>
__device__ __forceinline__ int decode_tiles_of_request(const FwdParams& p, int r) {
    const int ql = req_qend(p, r) - req_q0(p, r);
    return decode_tiles_of<VAR>(p, ql, req_L(p, r, ql));
}

// Wave index whose tile range holds global tile t (ranges [w N / W, (w+1) N / W)).
__device__ __forceinline__ int64_t wave_of_tile(int64_t t, int64_t N, int64_t W) { return ((t + 1) * W - 1) / N; }

// Position of a decode wave in the global tile list: request r, kv head kh,
// tile t of the (r, kh) item (key tile t0 + t of the request), global index
// T, with request r's tiles per item (n), first tile (t0), KV length (L) and
// query range (q0, q_len). An invalid cursor (past the wave's range) keeps
// pointing at the wave's last tile.
struct DecodeCursor {
    int64_t T;
    int r, kh, t, n, t0, L, q0, q_len;
    bool valid;
    __device__ __forceinline__ int key0() const { return (t0 + t) * kDecodeTile; }
};

// RB: blocks of 16 query rows per item (items of up to 16 RB rows); each
// block is a 16-column MFMA pass over the same K/V tile in LDS. With RB > 1
// the wave holds RB running states, every K and V fragment it reads feeds
// the MFMAs of all blocks (DecodeTile::compute_rows), and it may use the
// whole register file (one workgroup per CU).
// (bf16 tiles of head size 128 take 128 KB of LDS: one workgroup per CU)
template <int HD, bool FP8, bool PAGED, bool VAR, int RB>
__global__ __launch_bounds__(256, HD <= 128 && RB == 1 && (FP8 || HD != 128) ? 2 : 1) void decode_balanced_kernel(FwdParams p) {
    using DT = DecodeTile<HD, FP8>;
    constexpr int MB = DT::MB;
    constexpr int NL = DT::NL;
    constexpr int ROWS = 16 * RB;
    // tiles straight into LDS, two stages per wave (head size 128)
    constexpr bool DMA = DT::DMA;
    static_assert(!DMA || DT::NL * 1024 == DT::DMA_TILE, "one 1 KB copy per load");
    constexpr int SMEM = DMA ? 4 * 2 * DT::DMA_STAGE : 4 * DT::ELEMS * 2;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
    const int64_t gw = (int64_t)blockIdx.x * 4 + w;
    const int64_t W = (int64_t)gridDim.x * 4;

    // total tiles, then the request holding this wave's first tile; wave 0
    // also publishes the per-request tile prefix for the merge kernel
    int total = 0;
    for (int base = 0; base < p.B; base += 64) {
        int n = base + lane < p.B ? decode_tiles_of_request<VAR>(p, base + lane) : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
        total += __builtin_amdgcn_readfirstlane(n);
    }
    // (the scan results are the same in every lane; readfirstlane tells the
    // compiler so, which keeps the schedule and the loop below scalar)
    const int64_t N = (int64_t)p.Hkv * total;
    const int64_t T0 = gw * N / W, T1 = (gw + 1) * N / W;
    int r = -1, pr = 0, carry = 0;
    for (int base = 0; base < p.B; base += 64) {
        const int rr = base + lane;
        const int n = rr < p.B ? decode_tiles_of_request<VAR>(p, rr) : 0;
        int incl = n;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const int excl = carry + incl - n;
        if (gw == 0 && rr < p.B) p.sk_prefix[rr] = excl;
        const bool here = n > 0 && (int64_t)p.Hkv * excl <= T0 && T0 < (int64_t)p.Hkv * (excl + n);
        const uint64_t bal = __ballot(here);
        if (bal != 0 && r < 0) {
            const int src = __ffsll((unsigned long long)bal) - 1;
            r = base + src;
            pr = __builtin_amdgcn_readfirstlane(__shfl(excl, src));
        }
        carry += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    }
    if (gw == 0 && lane == 0) p.sk_prefix[p.B] = carry;
    if (T0 >= T1 || r < 0) return;

    // Request metadata window: lane j describes request wb + j.
    int wb = -1, w_n = 0, w_t0 = 0, w_L = 0, w_q0 = 0, w_ql = 0;
    auto fill = [&](DecodeCursor& c) {
        if (wb < 0 || c.r >= wb + 64) {
            wb = c.r;
            const int x = wb + lane;
            w_q0 = x < p.B ? req_q0(p, x) : 0;
            w_ql = x < p.B ? req_qend(p, x) - w_q0 : 0;
            w_L = x < p.B ? req_L(p, x, w_ql) : 0;
            w_n = decode_tiles_of<VAR>(p, w_ql, w_L);
            if constexpr (VAR) w_t0 = decode_first_tile<VAR>(p, w_ql, w_L);
        }
        const int j = __builtin_amdgcn_readfirstlane(c.r - wb);
        c.n = __builtin_amdgcn_readlane(w_n, j);
        if constexpr (VAR) c.t0 = __builtin_amdgcn_readlane(w_t0, j);
        else c.t0 = 0;
        c.L = __builtin_amdgcn_readlane(w_L, j);
        c.q0 = __builtin_amdgcn_readlane(w_q0, j);
        c.q_len = __builtin_amdgcn_readlane(w_ql, j);
    };
    // next tile of the wave's range (request-major, then kv head)
    auto advance = [&](DecodeCursor& c) {
        if (!c.valid) return;
        if (c.T + 1 >= T1) {
            c.valid = false;
            return;
        }
        const DecodeCursor prev = c;
        ++c.T;
        if (++c.t == c.n) {
            c.t = 0;
            if (++c.kh == p.Hkv) {
                c.kh = 0;
                do {
                    ++c.r;
                    fill(c);
                } while (c.n == 0 && c.r < p.B);
                if (c.r >= p.B) {  // only on metadata that contradicts itself
                    c = prev;
                    c.valid = false;
                }
            }
        }
    };

    DecodeCursor c0;
    c0.r = r;
    fill(c0);
    {
        const int64_t off = T0 - (int64_t)p.Hkv * pr;
        c0.kh = (int)(off / c0.n);
        c0.t = (int)(off % c0.n);
    }
    c0.T = T0;
    c0.valid = true;
    DecodeCursor c1 = c0;
    advance(c1);
    DecodeCursor c2 = c1;
    advance(c2);

    // Keys are clamped to the request's last key, so tiles that run past it
    // (and the re-read of the last tile past the wave's range) stay inside
    // the request's pages. Each lane translates the keys it loads itself.
    auto page_for = [&](const DecodeCursor& c, int (&pg)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int pos = min(c.key0() + DT::key_of(lane, i), c.L - 1);
            if constexpr (PAGED) pg[i] = req_bt(p, c.r)[page_index(pos, p.bs, p.bs_shift)];
            else pg[i] = c.q0 + pos;
        }
    };
    auto row_from = [&](const DecodeCursor& c, const int (&pg)[NL], int (&rows)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int pos = min(c.key0() + DT::key_of(lane, i), c.L - 1);
            if constexpr (PAGED) rows[i] = pg[i] * p.bs + page_offset(pos, p.bs, p.bs_shift);
            else rows[i] = pg[i];
        }
    };

    uint16_t* const stage = (uint16_t*)smem + w * DT::ELEMS;
    uint8_t* const dstage = smem + w * 2 * DT::DMA_STAGE;  // (DMA) stage 0, then stage 1
    float sl2 = p.scale_log2;
    if constexpr (FP8) sl2 *= *p.k_scale;
    const float vsc = FP8 ? *p.v_scale : 1.f;
    const int row = lane & 15;
    const int G = lane >> 4;

    // per row block rb (rows 16 rb + lane % 16): query fragment, key bounds,
    // sink logit (log2 domain, loaded with the item's query fragment) and
    // running softmax state
    // (one block prefetches the next item's query fragment with that item's
    // first tile; several blocks load it when the item starts, to keep
    // within the register file)
    constexpr bool QN = RB == 1;
    u32x4 qf[RB][DT::KS], qn[DT::KS];
    int limit[RB], lo[RB], qpos[RB];
    float sk[RB], sk_next[RB], m_run[RB], l_run[RB], lc_run[RB], al2[RB];
    f32x4 oacc[RB][MB];
    const bool has_sinks = p.sinks != nullptr;
    auto head_of = [&](int kh, int rb) { return kh * p.g + (16 * rb + row) % p.g; };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        load_decode_q<HD>(p, lane, c0.q0, c0.q_len * p.g, c0.kh, qf[rb], 16 * rb);
        limit[rb] = decode_row_limit(p, lane, c0.q_len, c0.L, req_causal(p, c0.r), 16 * rb);
        lo[rb] = VAR ? decode_row_lo(p, lane, c0.q_len, c0.L, 16 * rb) : 0;
        al2[rb] = VAR ? decode_row_alibi(p, lane, c0.kh, 16 * rb) : 0.f;
        qpos[rb] = decode_row_pos(p, lane, c0.q_len, c0.L, 16 * rb);
        sk[rb] = has_sinks ? sink_l2(p, head_of(c0.kh, rb)) : -INFINITY;
        sk_next[rb] = -INFINITY;
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
        lc_run[rb] = 0.f;
#pragma unroll
        for (int i = 0; i < MB; ++i) oacc[rb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int seg_t0 = c0.t;  // first tile of the current item segment

    // The end of an item segment, in two steps. close(): normalise the
    // running output in place (oacc *= 1/l) and form its lse. write(): store
    // it, as the final output when the segment is the whole item, else as a
    // partial state in slot (wave + item); then reset the running state.
    // write() runs at the top of the next iteration, before that iteration's
    // loads: its stores then retire behind nothing, and the wait for the
    // next tile's loads covers them at no cost. (Issued after the loads, the
    // stores would have to be waited for on their own, a stall at every item
    // boundary a wave crosses.)
    float w_lse[RB];
    bool w_whole = false;
    DecodeCursor wc = c0;
    auto close = [&](const DecodeCursor& c) {
        // (a cascade's partial states all go to the merge: none is final)
        w_whole = seg_t0 == 0 && c.t == c.n - 1 && p.casc_len == 0;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float l = l_run[rb], lc = lc_run[rb];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            lc += __shfl_xor(lc, 16);
            lc += __shfl_xor(lc, 32);
            // a sink joins the normaliser once: in the final output of a
            // whole item, else in the merge
            float inv;
            finalize_row(m_run[rb], l, lc, w_whole ? sk[rb] : -INFINITY, vsc, inv, w_lse[rb]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) oacc[rb][mb] *= inv;
        }
        wc = c;
    };
    auto write = [&]() {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r16 = 16 * rb + row;
            if (r16 < wc.q_len * p.g) {
                if (w_whole) {
                    const int64_t tok = wc.q0 + r16 / p.g;
                    const int head = head_of(wc.kh, rb);
                    uint16_t* op = (uint16_t*)p.out + (tok * p.H + head) * HD + G * 4;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        float v4[4] = {oacc[rb][mb][0], oacc[rb][mb][1], oacc[rb][mb][2], oacc[rb][mb][3]};
                        store_bf16<4>(op + mb * 16, v4);
                    }
                    if (p.lse && G == 0) p.lse[(int64_t)head * p.T + tok] = w_lse[rb];
                } else {
                    const int64_t slot = gw + (int64_t)wc.r * p.Hkv + wc.kh;
                    float* op = p.part_o + (slot * ROWS + r16) * HD + G * 4;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) *(f32x4*)(op + mb * 16) = oacc[rb][mb];
                    if (G == 0) p.part_lse[slot * ROWS + r16] = w_lse[rb];
                }
            }
            m_run[rb] = -INFINITY;
            l_run[rb] = 0.f;
            lc_run[rb] = 0.f;
#pragma unroll
            for (int i = 0; i < MB; ++i) oacc[rb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // One software pipeline over the wave's whole tile range, across item
    // boundaries: iteration i writes out the segment tile i-1 closed (if
    // any), requests the block-table entries of tile i+2, issues the K/V
    // loads of tile i+1 (and, when tile i+1 opens another item, that item's
    // query fragment), computes tile i from LDS, closes tile i's item segment
    // if it ends there, and moves tile i+1 into LDS. A new item therefore
    // costs no pipeline restart. Past the wave's range the last tile is
    // re-read (cached) and never computed.
    u32x4 kr[DMA ? 1 : NL], vr[DMA ? 1 : NL];
    int pg[NL], rows[NL];
    int par = 0;  // (DMA) stage of the tile being computed
    page_for(c0, pg);
    row_from(c0, pg, rows);
    page_for(c1, pg);
    if constexpr (DMA) DT::issue(p, lane, rows, c0.kh, dstage);
    else DT::load(p, lane, rows, c0.kh, kr, vr);
    row_from(c1, pg, rows);
    if constexpr (DMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    else DT::store(stage, lane, kr, vr);
    bool pending = false;
    while (true) {
        if (pending) write();
        pending = false;
        page_for(c2, pg);
        if constexpr (DMA) {
            wave_lds_sync();  // (the other stage's last reads are done)
            DT::issue(p, lane, rows, c1.kh, dstage + (par ^ 1) * DT::DMA_STAGE);
        } else {
            DT::load(p, lane, rows, c1.kh, kr, vr);
        }
        const bool c1_new = c1.valid && c1.t == 0;
        if constexpr (QN) {
            if (c1_new) {
                load_decode_q<HD>(p, lane, c1.q0, c1.q_len * p.g, c1.kh, qn);
                if (has_sinks) sk_next[0] = sink_l2(p, head_of(c1.kh, 0));
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch issued before the compute
        {
            // every block, rows or not (a block without rows keeps an empty
            // state): one instance of the computation per kernel, since
            // several, chosen by the item's row count, made the compiler
            // spill; the matrix work of empty blocks hides under the tile
            // loads
            const uint16_t* const tile = DMA ? (const uint16_t*)(dstage + par * DT::DMA_STAGE) : stage;
            DT::template compute_rows<VAR, DMA, RB, RB>(tile, lane, c0.key0(), lo, limit, sl2, p.softcap_l2,
                                                        p.softcap_inv2, al2, qpos, qf, m_run, l_run, lc_run, oacc);
        }
        if (!c1.valid || c1_new) {
            close(c0);
            pending = true;
        }
        if (!c1.valid) break;
        row_from(c2, pg, rows);
        c0 = c1;
        c1 = c2;
        advance(c2);
        if (c1_new) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if constexpr (QN) {
#pragma unroll
                    for (int ks = 0; ks < DT::KS; ++ks) qf[rb][ks] = qn[ks];
                    sk[rb] = sk_next[rb];
                } else {
                    // (the loads complete with this iteration's tile loads)
                    load_decode_q<HD>(p, lane, c0.q0, c0.q_len * p.g, c0.kh, qf[rb], 16 * rb);
                    sk[rb] = has_sinks ? sink_l2(p, head_of(c0.kh, rb)) : -INFINITY;
                }
                limit[rb] = decode_row_limit(p, lane, c0.q_len, c0.L, req_causal(p, c0.r), 16 * rb);
                if constexpr (VAR) {
                    lo[rb] = decode_row_lo(p, lane, c0.q_len, c0.L, 16 * rb);
                    al2[rb] = decode_row_alibi(p, lane, c0.kh, 16 * rb);
                }
                qpos[rb] = decode_row_pos(p, lane, c0.q_len, c0.L, 16 * rb);
            }
            seg_t0 = 0;
        }
        if constexpr (!DMA) DT::store(stage, lane, kr, vr);
        // Nothing may be left in flight here: the next iteration's loads are
        // then the only ones its waits count (the query loads would otherwise
        // make the compiler wait on every tile load it issues). With DMA this
        // is also where the next tile has landed in the other stage.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __builtin_amdgcn_sched_barrier(0);
        par ^= 1;
    }
    write();  // the wave's last segment
}

// ----------------------------------------------------------------- prefill

// K tiles kept as e4m3fn for the fp8 QK^T MFMA (head size 128): 128-byte
// rows, 1 KB copy groups of 8 rows with no padding, the 16-byte chunk c of
// row r at position c ^ sw(r). With this permutation the 16-byte A-operand
// reads (rows l % 32, chunks picked by l / 32) hit every one of the 64 LDS
// banks once per 16 lanes.
struct PfK8 {
    static constexpr int RP = 128;
    static __device__ __forceinline__ int sw(int r) { return 2 * ((r >> 1) & 1) ^ ((r >> 2) & 1) ^ 4 * ((r >> 3) & 1); }
};

// VAR: the sliding window / soft cap code is compiled in.
// Q8: q is e4m3fn (with q_scale) over an e4m3fn cache; S^T = K Q^T runs on
// the fp8 MFMA with K copied into LDS as bytes, PV stays on the bf16 MFMA
// (V widened to bf16, P rounded to bf16: an e4m3 P would cost up to about
// 2^-4 of a value row's magnitude per output element).
// KSPLIT: work items of 64 query rows (decode-shaped batches such as
// speculative verification): waves w and w + 2 hold the same 32 rows, wave
// w < 2 the first 32 keys of every tile and wave w + 2 the last 32, and at
// the end each pair folds its two running states by log-sum-exp through
// LDS. Each wave then does half the matrix and exponential work per tile,
// so an item's tiles pass twice as fast (the waves that a 128-row item of
// such a batch leaves without rows would otherwise compute nothing useful).
template <int HD, bool FP8, int PG, bool VAR, bool Q8, bool KSPLIT = false>
__global__ __launch_bounds__(256, HD <= 128 ? 2 : 1) void prefill_kernel(FwdParams p) {
    constexpr int NW = kPrefillWaves;           // waves per workgroup
    constexpr int ROWS = KSPLIT ? kPrefillSplitRows : prefill_rows(HD);  // query rows per work item
    constexpr int TILE = prefill_tile(HD);      // keys per tile
    constexpr int CPR = HD / 8;                 // 16-byte chunks per row
    using PT = PfTile<HD>;                      // LDS tile layout
    constexpr int KPI = 64 / CPR;               // keys per 64-lane copy (bf16)
    constexpr int CPW = TILE / KPI / NW;        // copies per wave per K or V tile (bf16)
    constexpr int FPR = HD / 16;                // 16-byte fp8 loads per cache row
    constexpr int FKPI = 64 / FPR;              // keys per 64-lane fp8 load
    constexpr int FCPW = TILE / FKPI / NW;      // fp8 loads per wave per tile
    constexpr int NK = FP8 ? FCPW : CPW;        // keys each lane translates per tile
    constexpr int KS = HD / 16;                 // k-steps of S^T = K Q^T (32x32x16)
    constexpr int MB = HD / 32;                 // 32-row blocks of O^T
    constexpr int KB = TILE / 32;               // 32-key blocks per tile
    constexpr int KBW = KSPLIT ? 1 : KB;        // 32-key blocks of a tile each wave computes
    constexpr int SLOT = TILE / PT::KPI * PT::GP;  // bytes of one K or V tile
    static_assert(TILE == kTileRows && CPW >= 1 && FCPW >= 1 && KPI == PT::KPI, "");
    static_assert(!Q8 || (FP8 && HD == 128 && FPR == 8), "the fp8 MFMA mode is built for head size 128");
    // K tile j in k_lds<j % 2>, V tile j in v_lds<j % 2>; four separate arrays
    // so that the compiler sees the copies into one slot are independent of
    // the reads of another and does not wait for them
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[SLOT];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = KSPLIT ? (w & 1) : w;       // the wave's group of 32 rows
    const int kbw0 = KSPLIT ? (w >> 1) : 0;    // the wave's first 32-key block of a tile
    // Work order. Workgroup id i runs on XCD i % 8; each (request, kv head)
    // stream is pinned to XCD stream % 8 and its query tiles take consecutive
    // slots there, longest (highest) tile first, so the workgroups that share
    // a stream's K/V run together under one L2.
    const int nrk = p.B * p.Hkv;
    const int xcd = (int)(blockIdx.x % kXcds);
    const int slot_x = (int)(blockIdx.x / kXcds);
    const int rk = (slot_x / p.n_qtiles) * kXcds + xcd;
    const int qt = p.n_qtiles - 1 - slot_x % p.n_qtiles;
    if (rk >= nrk) return;
    const int r = rk / p.Hkv, kh = rk % p.Hkv;
    const int s = blockIdx.y;
    const int g = p.g;
    const int q0 = req_q0(p, r);
    const int q_len = req_qend(p, r) - q0;
    const int tpw = ROWS / g;  // tokens per work item
    const int tok0 = qt * tpw;
    if (tok0 >= q_len) return;
    const int L = req_L(p, r, q_len);
    const int ctx = L - q_len;
    const int tok_last = min(q_len, tok0 + tpw) - 1;
    const int item_end = p.causal ? min(L, ctx + tok_last + 1) : L;
    // with a sliding window no row of the item sees a key below the window
    // of its first token (a split that lies wholly below it is never read)
    const int k_split = (VAR ? window_base(p, q_len, L) : 0) + (p.num_splits > 1 ? s * p.split_len : 0);
    const int k_begin = VAR ? max(k_split, window_lo(p, ctx + tok0) & ~(TILE - 1)) : k_split;
    const int k_end = p.num_splits > 1 ? min(item_end, k_split + p.split_len) : item_end;
    if (k_begin >= k_end) return;

    // this lane's query row
    const int hsel = lane >> 5;  // which half of the 32-row MFMA tile's k dimension this lane feeds
    const int rho = wr * kPrefillRowsPerWave + (lane & 31);
    const int tl = tok0 + rho / g;
    const bool row_ok = rho < tpw * g && tl < q_len;
    const int head = kh * g + rho % g;
    int limit = p.causal ? min(L, ctx + tl + 1) : L;
    limit = row_ok ? min(limit, k_end) : 0;
    const int lo = VAR ? window_lo(p, ctx + tl) : 0;  // first key the row sees
    // keys below wave_min are visible to every valid row of the wave: tiles
    // that end there need no mask (rows past the end of the request are never
    // stored, so their scores do not matter)
    const int wtok_first = tok0 + (wr * kPrefillRowsPerWave) / g;
    const bool wave_any = wtok_first < q_len && wr * kPrefillRowsPerWave < tpw * g;
    const int wave_min = !wave_any ? k_begin : (p.causal ? min(k_end, ctx + wtok_first + 1) : k_end);
    // with a sliding window, keys at or past wave_lo are visible to every
    // valid row of the wave: tiles that start there need no lower mask
    int wave_lo = 0;
    if (VAR && wave_any) {
        const int wrho_last = min(wr * kPrefillRowsPerWave + kPrefillRowsPerWave, tpw * g) - 1;
        wave_lo = window_lo(p, ctx + min(q_len - 1, tok0 + wrho_last / g));
    }

    u32x4 qf[KS];
    // Q8: bytes 64 ks + 32 hsel + 16 t of the row, t = 0, 1 (B operand of the
    // fp8 MFMA, k-steps of 64)
    constexpr int KS8 = HD / 64;
    u32x4 qf8[KS8][2];
    if constexpr (Q8) {
        const uint8_t* qp = (const uint8_t*)p.q + ((int64_t)(q0 + (row_ok ? tl : 0)) * p.H + head) * HD + hsel * 32;
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                qf8[ks][t] = row_ok ? *(const u32x4*)(qp + ks * 64 + t * 16) : u32x4{0u, 0u, 0u, 0u};
    } else {
        const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(q0 + (row_ok ? tl : 0)) * p.H + head) * HD + hsel * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? *(const u32x4*)(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    float sl2 = p.scale_log2, vsc = 1.f;
    if constexpr (FP8) {
        sl2 *= *p.k_scale;
        vsc = *p.v_scale;
    }
    if constexpr (Q8) sl2 *= *p.q_scale;
    // With the soft cap or ALiBi the scores are scaled, capped and biased in
    // place (log2 domain) before the mask, and the softmax then takes them
    // with scale 1.
    const float al2 = VAR ? alibi_l2(p, head) : 0.f;  // this row's ALiBi slope
    const int qpos = ctx + tl;                         // and its sequence position
    const bool capped = VAR && (p.softcap_l2 > 0.f || p.alibi);
    const float sl2_cap = sl2;
    if (capped) sl2 = 1.f;

    // Per-lane LDS read offsets. The chunk permutation only touches the bits
    // in SWMASK and depends on row bits 0..3, so the other chunk bits, the
    // key block and the row group of each read are immediates; one offset
    // per pattern of the masked chunk bits.
    // K fragment (kb, ks): row kb*32 + (lane & 31), chunk 2 ks + hsel.
    constexpr int KPAT = 1 << popcount((2 * (KS - 1)) & PT::SWMASK & ~1);
    uint32_t koffs[KPAT];
    {
        const int rk = lane & 31;
#pragma unroll
        for (int j = 0; j < KPAT; ++j) {
            // the masked chunk bits of pattern j (bit 0 is hsel's, never 2 ks's)
            int cm = 0, k = 0;
#pragma unroll
            for (int b = 1; b < 16; ++b)
                if (PT::SWMASK & ~1 & (1 << b)) cm |= ((j >> k++) & 1) << b;
            const int c_lane = cm | hsel;  // chunk bits that vary with the lane or the pattern
            koffs[j] = PT::row_base(rk) + ((c_lane & PT::SWMASK) ^ PT::sw(rk)) * 16 + (c_lane & ~PT::SWMASK) * 16;
        }
    }
    // transposed V read (k2, hi, mb): row 16 k2 + 8 hi + 4 hsel + (lane & 15) / 4,
    // chunk 4 mb + cp with cp = 2 ((lane >> 4) & 1) + (lane & 3) / 2, half
    // lane & 1. Row bit 3 (hi) enters the permutation only through A3.
    constexpr int VPAT = 1 << popcount((4 * (MB - 1)) & PT::SWMASK & ~3);
    constexpr int VHI = PfLayout<HD>::A3 ? 2 : 1;
    uint32_t voffs[VHI][VPAT];
    {
        const int cp = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int h = 0; h < VHI; ++h) {
            const int rv = 8 * h + 4 * hsel + ((lane & 15) >> 2);
#pragma unroll
            for (int j = 0; j < VPAT; ++j) {
                int cm = 0, k = 0;
#pragma unroll
                for (int b = 2; b < 16; ++b)
                    if (PT::SWMASK & ~3 & (1 << b)) cm |= ((j >> k++) & 1) << b;
                const int c_lane = cm | cp;
                voffs[h][j] = PT::row_base(rv) - (VHI == 2 && h ? PT::row_base(8) : 0) +
                              ((c_lane & PT::SWMASK) ^ PT::sw(rv)) * 16 + (c_lane & ~PT::SWMASK) * 16 + (lane & 1) * 8;
            }
        }
    }

    // Tile copies. bf16: copy jj of wave w moves keys (w CPW + jj) KPI ..
    // + KPI - 1, lane l the 16-byte chunk at position l % CPR of key
    // (w CPW + jj) KPI + l / CPR. fp8: load jj of wave w reads 16 cached
    // bytes (chunks 2q and 2q + 1, q = l % FPR) of key (w FCPW + jj) FKPI +
    // l / FPR, widened to bf16 in registers and stored. Keys are clamped to
    // the last key of the range, so rows past the end hold a real, finite key
    // that the mask removes.
    const int32_t* bt_row = p.bt ? p.bt + (int64_t)r * p.bt_stride : nullptr;
    constexpr int NP = PG == kPgAny ? NK : 1;   // block-table entries a lane holds per tile
    auto key_of = [&](int jj) -> int {
        if constexpr (FP8) return (w * FCPW + jj) * FKPI + lane / FPR;
        else return (w * CPW + jj) * KPI + lane / CPR;
    };
    // The cache rows of this lane's keys in the tile starting at t0 come in
    // two steps, so that the block-table reads can be issued an iteration
    // before their use: page_of reads the entries, row_of forms a row (the
    // host keeps num_blocks * block_size below 2^31).
    auto page_of = [&](int t0, int32_t (&pg)[NP]) {
        if constexpr (PG == kPgAny) {
#pragma unroll
            for (int jj = 0; jj < NK; ++jj) pg[jj] = bt_row[min(t0 + key_of(jj), k_end - 1) / p.bs];
        } else if constexpr (PG == kPgWide) {
            pg[0] = bt_row[min(t0 + 16 * w, k_end - 1) >> p.bs_shift];
        } else {
            pg[0] = 0;
        }
    };
    auto row_of = [&](int t0, const int32_t (&pg)[NP], int jj) -> int32_t {
        const int pos = min(t0 + key_of(jj), k_end - 1);
        if constexpr (PG == kPgAny) return pg[jj] * p.bs + pos % p.bs;
        else if constexpr (PG == kPgWide) return pg[0] * p.bs + (pos & (p.bs - 1));
        else return q0 + pos;
    };
    u32x4 st_k[NK], st_v[NK];  // fp8 staging
    // (Q8: K tiles go to LDS as bytes, copied like the bf16 tiles: load jj of
    // wave w moves keys (w FCPW + jj) FKPI .. + 7, 1 KB of whole rows)
    auto issue = [&](const void* cache, int t0, const int32_t (&pg)[NP], uint8_t* slot, u32x4 (&st)[NK],
                     bool k_tile) {
#pragma unroll
        for (int jj = 0; jj < NK; ++jj) {
            // first element of the key's head row
            const int64_t rowe = ((int64_t)row_of(t0, pg, jj) * p.Hkv + kh) * HD;
            if (Q8 && k_tile) {
                const int chunk = (lane % FPR) ^ PfK8::sw(key_of(jj));
                copy16_to_lds<0>((const uint8_t*)cache + rowe + chunk * 16, slot + (w * FCPW + jj) * 1024);
            } else if constexpr (FP8) {
                st[jj] = *(const u32x4*)((const uint8_t*)cache + rowe + (lane % FPR) * 16);
            } else {
                const int chunk = (lane % CPR) ^ PT::sw(key_of(jj));
                copy16_to_lds<0>((const uint16_t*)cache + rowe + chunk * 8, slot + (w * CPW + jj) * PT::GP);
            }
        }
    };
    // fp8: widen the staged bytes and store them at their permuted positions
    auto land = [&](uint8_t* slot, const u32x4 (&st)[NK]) {
#pragma unroll
        for (int jj = 0; jj < NK; ++jj) {
            const int key = key_of(jj), q = lane % FPR, sw = PT::sw(key);
            uint8_t* row = slot + PT::row_base(key);
            *(u32x4*)(row + ((2 * q) ^ sw) * 16) = fp8x8_to_bf16x8(u32x2{st[jj].x, st[jj].y});
            *(u32x4*)(row + ((2 * q + 1) ^ sw) * 16) = fp8x8_to_bf16x8(u32x2{st[jj].z, st[jj].w});
        }
    };

    float m_run = -INFINITY, l_run = 0.f, lc_run = 0.f;  // lc_run: sum of the bf16-rounded probabilities
    f32x16 oacc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;

    // Q8: per-lane byte offsets of the K fragment (row l % 32 of a 32-key
    // block, chunk 4 ks + 2 hsel + t at its permuted position)
    uint32_t koff8[KS8][2];
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            koff8[ks][t] = (lane & 31) * PfK8::RP + 16 * ((4 * ks + 2 * hsel + t) ^ PfK8::sw(lane & 31));
    // S^T = K Q^T for the wave's key blocks of one tile
    auto qk = [&](const uint8_t* kslot, f32x16 (&sacc)[KBW]) {
        if constexpr (KSPLIT) kslot += kbw0 * PT::row_base(32);
        if constexpr (Q8) {
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS8; ++ks)
                    sacc[kb] = mfma32x32x64_fp8(*(const u32x4*)(kslot + kb * 32 * PfK8::RP + koff8[ks][0]),
                                                *(const u32x4*)(kslot + kb * 32 * PfK8::RP + koff8[ks][1]),
                                                qf8[ks][0], qf8[ks][1], sacc[kb]);
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc[kb] = mfma32x32x16(
                    *(const u32x4*)(kslot + koffs[pext(2 * ks, PT::SWMASK & ~1)] + ((2 * ks) & ~PT::SWMASK) * 16 +
                                    kb * PT::row_base(32)),
                    qf[ks], sacc[kb]);
        }
    };
    // soft cap and ALiBi bias of the scores of the tile starting at key t0
    // (before the mask), taking them to the log2 domain
    auto cap = [&](int t0, f32x16 (&sacc)[KBW]) {
        t0 += kbw0 * 32;
        if (capped) {
            const bool sc = p.softcap_l2 > 0.f;
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float x = sacc[kb][e] * sl2_cap;
                    if (sc) x = softcap_l2(x, p.softcap_l2, p.softcap_inv2);
                    const int key = t0 + kb * 32 + (e >> 2) * 8 + (e & 3) + hsel * 4;
                    sacc[kb][e] = x - al2 * fabsf((float)(qpos - key));
                }
        }
    };
    // causal / length mask of a tile that reaches past wave_min, window mask
    // of one that starts below wave_lo
    auto mask = [&](int t0, f32x16 (&sacc)[KBW]) {
        t0 += kbw0 * 32;  // the wave's first key of the tile
        if (t0 + 32 * KBW > wave_min || (VAR && t0 < wave_lo)) {
            const int lim = limit - t0 - hsel * 4;
            const int low = lo - t0 - hsel * 4;
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int k = kb * 32 + (e >> 2) * 8 + (e & 3);
                    if (k >= lim || (VAR && k < low)) sacc[kb][e] = -INFINITY;
                }
        }
    };
    // row maximum of a tile (both lane halves hold keys of the same row)
    auto rowmax = [&](f32x16 (&sacc)[KBW]) -> float {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    // lazy rescale (wave-uniform decision)
    auto rescale = [&](float mx) {
        const float m_tile = mx * sl2;  // sl2 > 0: the scaled maximum
        if (__any(m_tile > m_run + kLazyRescale)) {
            const float m_new = fmaxf(m_run, m_tile);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
            lc_run *= alpha;
#pragma unroll
            for (int i = 0; i < MB; ++i) oacc[i] *= alpha;
            m_run = m_new;
        }
    };
    // probabilities of a tile as bf16 MFMA B operands, and their row sum
    auto expo = [&](f32x16 (&sacc)[KBW], u32x4 (&pf)[2 * KBW]) {
        const float nm = m_run == -INFINITY ? 0.f : -m_run;
        float ps = 0.f, pc = 0.f;
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
            float pv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                pv[e] = fast_exp2(fmaf(sacc[kb][e], sl2, nm));
                ps += pv[e];
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                pf[2 * kb + hf] = u32x4{pack_bf16x2(pv[8 * hf + 0], pv[8 * hf + 1]), pack_bf16x2(pv[8 * hf + 2], pv[8 * hf + 3]),
                                        pack_bf16x2(pv[8 * hf + 4], pv[8 * hf + 5]), pack_bf16x2(pv[8 * hf + 6], pv[8 * hf + 7])};
                const u32x4 w4 = pf[2 * kb + hf];
                pc = add_bf16_pair(w4.w, add_bf16_pair(w4.z, add_bf16_pair(w4.y, add_bf16_pair(w4.x, pc))));
            }
        }
        l_run += ps;
        lc_run += pc;
    };
    // O^T += V^T P^T for one tile
    auto pv = [&](const uint8_t* vslot, const u32x4 (&pf)[2 * KBW]) {
        if constexpr (KSPLIT) vslot += kbw0 * 2 * PT::row_base(16);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int k2 = 0; k2 < 2 * KBW; ++k2) {
                const int vj = pext(4 * mb, PT::SWMASK & ~3);
                const uint8_t* vp = vslot + ((4 * mb) & ~PT::SWMASK) * 16 + k2 * PT::row_base(16);
                const u32x2 lo = lds_read_tr16(vp + voffs[0][vj]);
                const u32x2 hi = lds_read_tr16(vp + voffs[VHI - 1][vj] + PT::row_base(8));
                oacc[mb] = mfma32x32x16(u32x4{lo.x, lo.y, hi.x, hi.y}, pf[k2], oacc[mb]);
            }
    };

    // Pipeline, tile i in iteration i. K tile j and V tile j are copied into
    // slot j % 2: K(i+2) and V(i+1) are issued at the start of iteration i and
    // land (barrier) at its end, so each copy has a whole iteration to arrive.
    // Inside the iteration the S^T MFMAs of tile i+1 and the PV MFMAs of tile
    // i are issued next to the exponentials of tile i, so the matrix cores
    // and the vector ALUs overlap; the mask of tile i+1, its row maximum and
    // the lazy-rescale decision for it follow, after PV, so that their
    // branches stay out of that block.
    const int n_tiles = (k_end - k_begin + TILE - 1) / TILE;
    f32x16 s_a[KBW], s_b[KBW];
    float mx;
    int32_t pg_v[NP];  // block-table entries of this lane's keys in tile i+1 (for V(i+1))
    int32_t pg_k[NP];  // block-table entries of this lane's keys in tile i+2 (for K(i+2))
    {
        int32_t pg0[NP];
        page_of(k_begin, pg0);
        issue(p.k_cache, k_begin, pg0, k_lds0, st_k, true);
        issue(p.v_cache, k_begin, pg0, v_lds0, st_v, false);
        if constexpr (FP8) {
            if constexpr (!Q8) land(k_lds0, st_k);  // (waits for its loads)
            land(v_lds0, st_v);
        }
        page_of(k_begin + TILE, pg_v);
        if (n_tiles > 1) {
            issue(p.k_cache, k_begin + TILE, pg_v, k_lds1, st_k, true);
            if constexpr (FP8 && !Q8) land(k_lds1, st_k);
        }
        page_of(k_begin + 2 * TILE, pg_k);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        qk(k_lds0, s_a);
        cap(k_begin, s_a);
        mask(k_begin, s_a);
        mx = rowmax(s_a);
        rescale(mx);
        __syncthreads();
    }
    auto iteration = [&](auto par, auto last, int i, f32x16 (&sc)[KBW], f32x16 (&sn)[KBW]) {
        constexpr int P = decltype(par)::value;
        constexpr bool LAST = decltype(last)::value;
        uint8_t* const k_here = P ? k_lds1 : k_lds0;   // K(i), now free: receives K(i+2)
        uint8_t* const k_next = P ? k_lds0 : k_lds1;   // K(i+1)
        uint8_t* const v_here = P ? v_lds1 : v_lds0;   // V(i)
        uint8_t* const v_next = P ? v_lds0 : v_lds1;   // receives V(i+1)
        const int t0 = k_begin + i * TILE;
        const bool load_k = i + 2 < n_tiles;
        int32_t pg_kk[NP];  // entries of tile i+2: V(i+2) is issued from them next iteration
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) pg_kk[jj] = pg_k[jj];
        if constexpr (!LAST) {
            if (load_k) issue(p.k_cache, t0 + 2 * TILE, pg_k, k_here, st_k, true);
            issue(p.v_cache, t0 + TILE, pg_v, v_next, st_v, false);
            if (i + 3 < n_tiles) page_of(t0 + 3 * TILE, pg_k);
        }
        u32x4 pf[2 * KBW];
        if constexpr (!LAST) qk(k_next, sn);
        expo(sc, pf);
        pv(v_here, pf);
        if constexpr (!LAST) {
            // (the mask branch comes after PV so that the S^T MFMAs of tile
            // i+1, the exponentials and the PV MFMAs of tile i share one
            // basic block for the scheduler)
            cap(t0 + TILE, sn);
            mask(t0 + TILE, sn);
            mx = rowmax(sn);
            rescale(mx);  // (here rather than before the exponentials: its branch stays out of that block)
            if constexpr (FP8) {
                if (!Q8 && load_k) land(k_here, st_k);
                land(v_next, st_v);
            }
#pragma unroll
            for (int jj = 0; jj < NP; ++jj) pg_v[jj] = pg_kk[jj];
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int i = 0;
    for (; i + 2 < n_tiles; i += 2) {
        iteration(I0{}, std::false_type{}, i, s_a, s_b);
        iteration(I1{}, std::false_type{}, i + 1, s_b, s_a);
    }
    if (n_tiles - i == 2) {
        iteration(I0{}, std::false_type{}, i, s_a, s_b);
        iteration(I1{}, std::true_type{}, i + 1, s_b, s_a);
    } else {
        iteration(I0{}, std::true_type{}, i, s_a, s_b);
    }

    if constexpr (KSPLIT) {
        // Waves 2 and 3 hand their running state (output accumulators in
        // a K slot, m / l / lc in a V slot, lane-contiguous) to the wave
        // that holds the same rows, which folds both by log-sum-exp; the
        // tile slots are free once every wave is past the loop.
        static_assert(MB * 16 * 64 * 4 <= SLOT && 3 * 64 * 4 <= SLOT, "the pair's state fits one slot");
        __syncthreads();
        float* const po = (float*)(wr ? k_lds1 : k_lds0);
        float* const ps = (float*)(wr ? v_lds1 : v_lds0);
        if (w >= 2) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) po[(mb * 16 + e) * 64 + lane] = oacc[mb][e];
            ps[lane] = m_run;
            ps[64 + lane] = l_run;
            ps[128 + lane] = lc_run;
        }
        __syncthreads();
        if (w >= 2) return;
        const float mb_ = ps[lane], lb = ps[64 + lane], lcb = ps[128 + lane];
        const float m_new = fmaxf(m_run, mb_);
        const float mr = m_new == -INFINITY ? 0.f : m_new;
        const float a = fast_exp2(m_run - mr), b = fast_exp2(mb_ - mr);  // 0 for a side with no key yet
        l_run = a * l_run + b * lb;
        lc_run = a * lc_run + b * lcb;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[mb][e] = a * oacc[mb][e] + b * po[(mb * 16 + e) * 64 + lane];
        m_run = m_new;
    }
    if (!row_ok) return;
    l_run += __shfl_xor(l_run, 32);
    lc_run += __shfl_xor(lc_run, 32);
    // a sink joins the normaliser once, in the final output
    float inv, lse;
    finalize_row(m_run, l_run, lc_run, p.num_splits == 1 ? sink_l2(p, head) : -INFINITY, vsc, inv, lse);
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
    const int r = request_of(p, tok);
    const int q0 = req_q0(p, r);
    const int q_len = req_qend(p, r) - q0;
    const int t = (int)(tok - q0);
    const int L = req_L(p, r, q_len);
    const int n_vis = p.causal ? max(0, min(L, L - q_len + t + 1)) : L;
    const int k_split = window_base(p, q_len, L) + (p.num_splits > 1 ? s * p.split_len : 0);
    const int k_end = p.num_splits > 1 ? min(n_vis, k_split + p.split_len) : n_vis;
    if (p.num_splits > 1 && k_split >= n_vis) return;
    const int k_begin = max(k_split, window_lo(p, L - q_len + t));
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
        const int64_t base = (int64_t)kv_row(bt_row, j, p.bs, p.bs_shift, q0) * rstride + (int64_t)kh * hd;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = lane + 64 * i;
            if (d < hd) dot += qv[i] * load_kv1<KV>(p.k_cache, base + d);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
        float x = dot * sl2;
        if (p.softcap_l2 > 0.f) x = softcap_l2(x, p.softcap_l2, p.softcap_inv2);
        if (p.alibi) x -= alibi_l2(p, h) * fabsf((float)(L - q_len + t - j));
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
    float inv, lse;
    finalize_row(m, l, p.num_splits == 1 ? sink_l2(p, h) : -INFINITY, vsc, inv, lse);
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

// Merge of the split partials. Split s of a row holds keys
// [base + s * split_len, base + (s+1) * split_len) (base: the request's
// window base, 0 without a window). The splits that hold the row's visible
// keys [lo, n_vis) are s_lo = (lo - base) / split_len up to
// ceil((n_vis - base) / split_len) - 1; every kernel writes at least those,
// and only those are read. A sink logit joins the normaliser here.
// One half-wave (32 lanes) per (token, head) row: lane j first holds the lse
// of splits j, j+32, ... and their weights, then the lanes accumulate
// 4-element chunks of the row over all splits, with independent loads.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
    constexpr int MAXC = 8;  // up to 256 splits, 32 per lane-chunk
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const int64_t rowi = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
    if (rowi >= p.T * p.H) return;  // whole half-waves leave together
    const int64_t tok = rowi / p.H;
    const int h = (int)(rowi % p.H);
    const int r = request_of(p, tok);
    const int q0 = req_q0(p, r);
    const int q_len = req_qend(p, r) - q0;
    const int L = req_L(p, r, q_len);
    const int t = (int)(tok - q0);
    const int n_vis = p.causal ? max(0, min(L, L - q_len + t + 1)) : L;
    const int base = window_base(p, q_len, L);
    const int s_lo = max(0, window_lo(p, L - q_len + t) - base) / p.split_len;
    const int s_end = min(p.num_splits, max(0, n_vis - base + p.split_len - 1) / p.split_len);
    const int n_valid = max(0, s_end - s_lo);  // splits s_lo + j, j < n_valid
    const int nc = (n_valid + 31) >> 5;
    float ls[MAXC];
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int sp = s_lo + c * 32 + hl;
        ls[c] = (c < nc && c * 32 + hl < n_valid) ? p.part_lse[((int64_t)sp * p.H + h) * p.T + tok] : -INFINITY;
        M = fmaxf(M, ls[c]);
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float wsum = 0.f;
    const float Mu = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        ls[c] = fast_exp2((ls[c] - Mu) * kLog2e);  // weight of split c*32 + hl (0 if absent)
        wsum += ls[c];
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
    float inv, lse;
    finalize_row(Mu * kLog2e, wsum, sink_l2(p, h), 1.f, inv, lse);
    const int nch = p.hd / 4;  // 4-element chunks per row (<= 64)
    const int base_lane = lane & 32;
    for (int cc = hl; cc < ((nch + 31) & ~31); cc += 32) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < nc; ++c) {
            const int cnt = min(32, n_valid - c * 32);
            for (int j = 0; j < cnt; ++j) {
                const float wgt = __shfl(ls[c], base_lane + j);
                const int sp = s_lo + c * 32 + j;
                if (cc < nch) o += wgt * *(const f32x4*)(p.part_o + (((int64_t)sp * p.T + tok) * p.H + h) * p.hd + 4 * cc);
            }
        }
        if (cc < nch) {
            o *= inv;
            const int64_t e = (tok * p.H + h) * p.hd + 4 * cc;
            if (OUT_F32) *(f32x4*)((float*)p.out + e) = o;
            else *(u32x2*)((uint16_t*)p.out + e) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
    }
    if (p.lse && hl == 0) p.lse[(int64_t)h * p.T + tok] = lse;
}

// Merge for the balanced decode schedule: one half-wave per row of a
// (request, kv head) item, merge_rows / 8 workgroups of eight half-waves per
// item (merge_rows: the batch's longest request's rows, at most the slot's
// 16 RB rows). The item was covered by waves wave_of(first tile) ..
// wave_of(last tile) (those that own at least one tile); with one wave the
// output is already final. The item comes from the block index, so the
// metadata loads are independent of each other.
// CH: partials read per chunk: 16 for items covered by many waves (long
// contexts), 4 otherwise (fewer registers, higher occupancy).
template <int CH>
__global__ __launch_bounds__(256) void combine_balanced_kernel(FwdParams p) {
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const int wgs = p.merge_rows >> 3;  // workgroups per item
    const int64_t item = blockIdx.x / wgs;
    const int r = (int)(item / p.Hkv);
    const int kh = (int)(item % p.Hkv);
    const int row16 = (int)((blockIdx.x % wgs) * 8 + (threadIdx.x >> 5));  // row within the item
    const int q0 = req_q0(p, r);
    const int q_len = req_qend(p, r) - q0;
    if (row16 >= q_len * p.g) return;  // whole half-waves leave together
    const int L = req_L(p, r, q_len);
    const int64_t N = (int64_t)p.Hkv * p.sk_prefix[p.B];
    const int64_t first = (int64_t)p.Hkv * p.sk_prefix[r];
    const int n_r = decode_tiles_of(p, q_len, L);
    const int64_t W = p.sk_waves;
    const int64_t g0 = first + (int64_t)kh * n_r;
    const int64_t wf = wave_of_tile(g0, N, W), wl = wave_of_tile(g0 + n_r - 1, N, W);
    if (wf == wl) return;
    const int64_t tok = q0 + row16 / p.g;
    const int h = kh * p.g + row16 % p.g;
    const int64_t slot0 = wf + item;
    const int np = (int)(wl - wf + 1);
    // with more waves than tiles some waves own no tile and wrote nothing
    auto owns_tiles = [&](int64_t w) { return (w + 1) * N / W > w * N / W; };
    const int nch = p.hd / 4;
    const bool c0 = hl < nch, c1 = hl + 32 < nch;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 o0 = zero, o1 = zero;
    float wsum = 0.f;
    // Partials in chunks of CH whose lse and output loads are issued
    // together (they depend only on the slot), with a running maximum
    // between chunks: about np / CH dependent round trips. Lane hl < CH
    // of each half-wave reads the lse of partial j0 + hl (and decides
    // whether it exists); the others take it by a lane shuffle.
    float M = -INFINITY;
    for (int j0 = 0; j0 < np; j0 += CH) {
        const int jl = j0 + hl;
        const float lsl = hl < CH && jl < np && owns_tiles(wf + jl)
                              ? p.part_lse[(slot0 + jl) * p.dec_rows + row16] : -INFINITY;
        float ls[CH];
        f32x4 v0[CH], v1[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            ls[u] = __shfl(lsl, (lane & 32) + u);
            v0[u] = zero;
            v1[u] = zero;
            if (j0 + u < np) {  // (np is the same for every lane of the wave)
                const float* src = p.part_o + ((slot0 + j0 + u) * p.dec_rows + row16) * p.hd;
                if (c0) v0[u] = *(const f32x4*)(src + 4 * hl);
                if (c1) v1[u] = *(const f32x4*)(src + 4 * (hl + 32));
            }
        }
        float cm = M;
#pragma unroll
        for (int u = 0; u < CH; ++u) cm = fmaxf(cm, ls[u]);
        if (cm == -INFINITY) continue;  // no partial yet
        const float a = fast_exp2((M - cm) * kLog2e);  // 0 while nothing is accumulated
        o0 *= a;
        o1 *= a;
        wsum *= a;
        M = cm;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const float wj = fast_exp2((ls[u] - M) * kLog2e);  // 0 for absent partials
            wsum += wj;
            // an absent partial's slot holds stale bytes: select, never multiply by 0
            if (wj != 0.f) {
                o0 += wj * v0[u];
                o1 += wj * v1[u];
            }
        }
    }
    const float Mu = M == -INFINITY ? 0.f : M;
    float inv, lse;
    finalize_row(Mu * kLog2e, wsum, sink_l2(p, h), 1.f, inv, lse);
    uint16_t* dst = (uint16_t*)p.out + (tok * p.H + h) * p.hd;
    if (c0) {
        o0 *= inv;
        *(u32x2*)(dst + 4 * hl) = u32x2{pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3])};
    }
    if (c1) {
        o1 *= inv;
        *(u32x2*)(dst + 4 * (hl + 32)) = u32x2{pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
    }
    if (p.lse && hl == 0) p.lse[(int64_t)h * p.T + tok] = lse;
}

// Merge for a cascade run as one balanced decode (casc_len > 0): request 0
// of the decode list is every token against the shared prefix, request r >= 1
// is request r - 1 against its own keys, and every segment left a partial
// state. One half-wave per row of a suffix item (request r >= 1, kv head kh):
// it folds the partials of that item and those of the prefix item (request 0,
// the same kv head) at the row of the same token and head, by log-sum-exp,
// and adds a sink logit to the normaliser once.
template <int CH>
__global__ __launch_bounds__(256) void combine_cascade_kernel(FwdParams p) {
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const int wgs = p.merge_rows >> 3;  // workgroups per item
    const int64_t sitem = blockIdx.x / wgs;
    const int r = 1 + (int)(sitem / p.Hkv);
    const int kh = (int)(sitem % p.Hkv);
    const int row16 = (int)((blockIdx.x % wgs) * 8 + (threadIdx.x >> 5));
    const int q0 = req_q0(p, r);
    const int q_len = req_qend(p, r) - q0;
    if (row16 >= q_len * p.g) return;  // whole half-waves leave together
    const int64_t tok = q0 + row16 / p.g;
    const int h = kh * p.g + row16 % p.g;
    const int64_t N = (int64_t)p.Hkv * p.sk_prefix[p.B];
    const int64_t W = p.sk_waves;
    auto owns_tiles = [&](int64_t w) { return (w + 1) * N / W > w * N / W; };
    const int nch = p.hd / 4;
    const bool c0 = hl < nch, c1 = hl + 32 < nch;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 o0 = zero, o1 = zero;
    float wsum = 0.f, M = -INFINITY;
    // the prefix item's row of this token and head, then this row of the suffix item
#pragma unroll 1
    for (int part = 0; part < 2; ++part) {
        const int rr = part == 0 ? 0 : r;
        const int row = part == 0 ? (int)(tok * p.g + row16 % p.g) : row16;
        const int ql = req_qend(p, rr) - req_q0(p, rr);
        const int n = decode_tiles_of(p, ql, req_L(p, rr, ql));
        if (n == 0) continue;
        const int64_t item = (int64_t)rr * p.Hkv + kh;
        const int64_t g0 = (int64_t)p.Hkv * p.sk_prefix[rr] + (int64_t)kh * n;
        const int64_t wf = wave_of_tile(g0, N, W), wl = wave_of_tile(g0 + n - 1, N, W);
        const int64_t slot0 = wf + item;
        const int np = (int)(wl - wf + 1);
        for (int j0 = 0; j0 < np; j0 += CH) {
            const int jl = j0 + hl;
            const float lsl = hl < CH && jl < np && owns_tiles(wf + jl)
                                  ? p.part_lse[(slot0 + jl) * p.dec_rows + row] : -INFINITY;
            float ls[CH];
            f32x4 v0[CH], v1[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                ls[u] = __shfl(lsl, (lane & 32) + u);
                v0[u] = zero;
                v1[u] = zero;
                if (j0 + u < np) {
                    const float* src = p.part_o + ((slot0 + j0 + u) * p.dec_rows + row) * p.hd;
                    if (c0) v0[u] = *(const f32x4*)(src + 4 * hl);
                    if (c1) v1[u] = *(const f32x4*)(src + 4 * (hl + 32));
                }
            }
            float cm = M;
#pragma unroll
            for (int u = 0; u < CH; ++u) cm = fmaxf(cm, ls[u]);
            if (cm == -INFINITY) continue;
            const float a = fast_exp2((M - cm) * kLog2e);
            o0 *= a;
            o1 *= a;
            wsum *= a;
            M = cm;
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const float wj = fast_exp2((ls[u] - M) * kLog2e);
                wsum += wj;
                if (wj != 0.f) {  // an absent partial's slot holds stale bytes
                    o0 += wj * v0[u];
                    o1 += wj * v1[u];
                }
            }
        }
    }
    const float Mu = M == -INFINITY ? 0.f : M;
    float inv, lse;
    finalize_row(Mu * kLog2e, wsum, sink_l2(p, h), 1.f, inv, lse);
    uint16_t* dst = (uint16_t*)p.out + (tok * p.H + h) * p.hd;
    if (c0) {
        o0 *= inv;
        *(u32x2*)(dst + 4 * hl) = u32x2{pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3])};
    }
    if (c1) {
        o1 *= inv;
        *(u32x2*)(dst + 4 * (hl + 32)) = u32x2{pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
    }
    if (p.lse && hl == 0) p.lse[(int64_t)h * p.T + tok] = lse;
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

// The decode kernels are built with and without the window / soft cap code.
static bool uses_var(const FwdParams& p) { return p.window_left >= 0 || p.softcap_l2 > 0.f || p.alibi; }
template <typename K1, typename K0>
static void launch_var(K1 with_var, K0 plain, bool var, dim3 grid, hipStream_t s, const FwdParams& p) {
    if (var) hipLaunchKernelGGL(with_var, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(plain, grid, dim3(256), 0, s, p);
}

template <int HD>
static hipError_t decode_hd(const FwdParams& p, KvType kv, hipStream_t s) {
    dim3 grid(p.num_splits, p.Hkv, p.B);
    const bool var = uses_var(p);
    const bool paged = p.bt != nullptr;
    if (kv == KvType::FP8) {
        if (paged) launch_var((decode_kernel<HD, true, true, true>), (decode_kernel<HD, true, true, false>), var, grid, s, p);
        else launch_var((decode_kernel<HD, true, false, true>), (decode_kernel<HD, true, false, false>), var, grid, s, p);
    } else {
        if (paged) launch_var((decode_kernel<HD, false, true, true>), (decode_kernel<HD, false, true, false>), var, grid, s, p);
        else launch_var((decode_kernel<HD, false, false, true>), (decode_kernel<HD, false, false, false>), var, grid, s, p);
    }
    return hipGetLastError();
}

template <int HD, int RB>
static void decode_balanced_rb(const FwdParams& p, KvType kv, bool var, dim3 grid, hipStream_t s) {
    const bool paged = p.bt != nullptr;
    if (kv == KvType::FP8) {
        if (paged) launch_var((decode_balanced_kernel<HD, true, true, true, RB>),
                              (decode_balanced_kernel<HD, true, true, false, RB>), var, grid, s, p);
        else launch_var((decode_balanced_kernel<HD, true, false, true, RB>),
                        (decode_balanced_kernel<HD, true, false, false, RB>), var, grid, s, p);
    } else {
        if (paged) launch_var((decode_balanced_kernel<HD, false, true, true, RB>),
                              (decode_balanced_kernel<HD, false, true, false, RB>), var, grid, s, p);
        else launch_var((decode_balanced_kernel<HD, false, false, true, RB>),
                        (decode_balanced_kernel<HD, false, false, false, RB>), var, grid, s, p);
    }
}

template <int HD>
static hipError_t decode_balanced_hd(const FwdParams& p, KvType kv, hipStream_t s) {
    dim3 grid(p.sk_waves / 4);
    const bool var = uses_var(p);
    if (p.dec_rows == 16) {
        decode_balanced_rb<HD, 1>(p, kv, var, grid, s);
    } else if constexpr (HD <= kDecodeMaxRbHead) {
        if (p.dec_rows == 32) decode_balanced_rb<HD, 2>(p, kv, var, grid, s);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_balanced(const FwdParams& p, KvType kv, hipStream_t s) {
    switch (p.hd) {
        case 64: return decode_balanced_hd<64>(p, kv, s);
        case 128: return decode_balanced_hd<128>(p, kv, s);
        case 256: return decode_balanced_hd<256>(p, kv, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine_balanced(const FwdParams& p, hipStream_t s) {
    const int64_t items = (int64_t)p.B * p.Hkv;  // merge_rows / 8 workgroups per item
    const dim3 grid((unsigned)(items * (p.merge_rows / 8)));
    // waves per item when all items are as long as the longest: chunks of
    // 16 partials pay off from about 16 partials per item
    if (p.sk_waves >= 16 * items) hipLaunchKernelGGL(combine_balanced_kernel<16>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(combine_balanced_kernel<4>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_combine_cascade(const FwdParams& p, hipStream_t s) {
    const int64_t items = (int64_t)(p.B - 1) * p.Hkv;  // suffix items; merge_rows / 8 workgroups each
    const dim3 grid((unsigned)(items * (p.merge_rows / 8)));
    if (p.sk_waves >= 16 * items) hipLaunchKernelGGL(combine_cascade_kernel<16>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(combine_cascade_kernel<4>, grid, dim3(256), 0, s, p);
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
static hipError_t prefill_hd(const FwdParams& p, KvType kv, bool q8, hipStream_t s) {
    const int64_t streams_per_xcd = ((int64_t)p.B * p.Hkv + kXcds - 1) / kXcds;
    dim3 grid((unsigned)(streams_per_xcd * kXcds * p.n_qtiles), p.num_splits);  // 64 * kPrefillWaves threads each
    const int pg = !p.bt ? kPgFlat : (p.bs_shift >= 4 ? kPgWide : kPgAny);
    const bool var = uses_var(p);
    if constexpr (HD == 128) {
        if (q8) {  // e4m3fn q over an e4m3fn cache
            if (kv != KvType::FP8) return hipErrorInvalidValue;
            if (pg == kPgFlat) launch_var((prefill_kernel<HD, true, kPgFlat, true, true>), (prefill_kernel<HD, true, kPgFlat, false, true>), var, grid, s, p);
            else if (pg == kPgWide) launch_var((prefill_kernel<HD, true, kPgWide, true, true>), (prefill_kernel<HD, true, kPgWide, false, true>), var, grid, s, p);
            else launch_var((prefill_kernel<HD, true, kPgAny, true, true>), (prefill_kernel<HD, true, kPgAny, false, true>), var, grid, s, p);
            return hipGetLastError();
        }
    }
    if (q8) return hipErrorInvalidValue;
    if (p.pf_ksplit) {  // items of 64 rows over a paged cache, head size <= 128
        if constexpr (HD <= 128) {
            if (pg == kPgFlat) return hipErrorInvalidValue;
            if (kv == KvType::FP8) {
                if (pg == kPgWide) launch_var((prefill_kernel<HD, true, kPgWide, true, false, true>), (prefill_kernel<HD, true, kPgWide, false, false, true>), var, grid, s, p);
                else launch_var((prefill_kernel<HD, true, kPgAny, true, false, true>), (prefill_kernel<HD, true, kPgAny, false, false, true>), var, grid, s, p);
            } else {
                if (pg == kPgWide) launch_var((prefill_kernel<HD, false, kPgWide, true, false, true>), (prefill_kernel<HD, false, kPgWide, false, false, true>), var, grid, s, p);
                else launch_var((prefill_kernel<HD, false, kPgAny, true, false, true>), (prefill_kernel<HD, false, kPgAny, false, false, true>), var, grid, s, p);
            }
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (kv == KvType::FP8) {
        if (pg == kPgFlat) launch_var((prefill_kernel<HD, true, kPgFlat, true, false>), (prefill_kernel<HD, true, kPgFlat, false, false>), var, grid, s, p);
        else if (pg == kPgWide) launch_var((prefill_kernel<HD, true, kPgWide, true, false>), (prefill_kernel<HD, true, kPgWide, false, false>), var, grid, s, p);
        else launch_var((prefill_kernel<HD, true, kPgAny, true, false>), (prefill_kernel<HD, true, kPgAny, false, false>), var, grid, s, p);
    } else {
        if (pg == kPgFlat) launch_var((prefill_kernel<HD, false, kPgFlat, true, false>), (prefill_kernel<HD, false, kPgFlat, false, false>), var, grid, s, p);
        else if (pg == kPgWide) launch_var((prefill_kernel<HD, false, kPgWide, true, false>), (prefill_kernel<HD, false, kPgWide, false, false>), var, grid, s, p);
        else launch_var((prefill_kernel<HD, false, kPgAny, true, false>), (prefill_kernel<HD, false, kPgAny, false, false>), var, grid, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_prefill(const FwdParams& p, KvType kv, bool q8, hipStream_t s) {
    switch (p.hd) {
        case 64: return prefill_hd<64>(p, kv, q8, s);
        case 128: return prefill_hd<128>(p, kv, q8, s);
        case 256: return prefill_hd<256>(p, kv, q8, s);
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
    const int64_t n = p.T * p.H * 32;  // a half-wave per (token, head) row
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
