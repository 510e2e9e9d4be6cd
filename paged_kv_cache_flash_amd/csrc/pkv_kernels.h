// pkv_kernels.h -- internal interface between the host API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Everything a forward kernel needs, passed by value as the kernel argument.
struct FwdParams {
    const void* q;            // [T, H, hd] (bf16 or f32)
    const void* k_cache;      // paged [num_blocks, bs, Hkv, hd] or flat [T, Hkv, hd]
    const void* v_cache;
    void* out;                // [T, H, hd], type of q
    float* lse;               // [H, T] or nullptr
    float* part_o;            // split partials [S, T, H, hd] fp32 (S > 1)
    float* part_lse;          // [S, H, T] fp32
    const int32_t* qsl;       // [B+1]
    const int32_t* seq_lens;  // [B] or nullptr (flat)
    const int32_t* bt;        // block table or nullptr (flat)
    const float* k_scale;     // fp8 only
    const float* v_scale;
    const float* q_scale;     // e4m3fn q only
    int64_t bt_stride;
    int64_t T;
    int32_t B, H, Hkv, g, hd, bs;
    int32_t bs_shift;         // log2(bs) when bs is a power of two, else -1
    int32_t num_splits;       // >= 1
    int32_t split_len;        // keys per split (multiple of the key tile) when num_splits > 1
    int32_t n_qtiles;         // prefill: query tiles per (request, kv head)
    int32_t causal;
    float scale_log2;         // softmax_scale * log2(e)
    // balanced decode schedule
    int32_t sk_waves;         // waves sharing the decode tiles (grid = sk_waves / 4 workgroups)
    int32_t* sk_prefix;       // [B+1] per-request tile prefix and total, written by the attention kernel
    int32_t dec_rows;         // query rows per item slot (16 or 32: 16-row blocks per item)
    int32_t pf_ksplit;        // prefill kernel: items of kPrefillSplitRows rows, two waves per 32 rows
    int32_t merge_rows;       // rows per item the merge covers: max_seqlen_q x group, rounded up to 8, <= dec_rows
    // attention variants
    int32_t window_left;      // < 0: no sliding window
    float softcap_l2;         // softcap * log2(e) (> 0), or 0: no soft cap
    float softcap_inv2;       // 2 / softcap (soft cap on)
    const float* sinks;       // [H] natural-log sink logits, or nullptr
    const float* alibi;       // [H] ALiBi slopes, or nullptr
    // cascade passes
    int32_t single_len;       // > 0: the batch is one request of all T tokens with this KV
                              // length (qsl and seq_lens are not read; B == 1)
    int32_t seq_off;          // keys before this index belong to another pass: request r's
                              // KV length is max(0, seq_lens[r] - seq_off), and the block
                              // table passed in starts at that key's page
    int32_t casc_len;         // > 0: both cascade passes in one balanced decode launch. Request 0
                              // is every token against the first casc_len keys of block-table
                              // row 0, with no causal mask; request r >= 1 is request r - 1
                              // against its own keys from casc_len on. B counts both.
};

// Request metadata as every kernel reads it (cascade passes included).
__device__ __forceinline__ int req_q0(const FwdParams& p, int r) {
    if (p.casc_len > 0) return r == 0 ? 0 : p.qsl[r - 1];
    return p.single_len > 0 ? 0 : p.qsl[r];
}
__device__ __forceinline__ int req_qend(const FwdParams& p, int r) {
    if (p.casc_len > 0) return r == 0 ? (int)p.T : p.qsl[r];
    return p.single_len > 0 ? (int)p.T : p.qsl[r + 1];
}
// KV length of request r with q_len query tokens (q_len itself in the flat layout).
__device__ __forceinline__ int req_L(const FwdParams& p, int r, int q_len) {
    if (p.casc_len > 0) return r == 0 ? p.casc_len : max(0, p.seq_lens[r - 1] - p.casc_len);
    if (p.single_len > 0) return p.single_len;
    return p.seq_lens ? max(0, p.seq_lens[r] - p.seq_off) : q_len;
}
// Block-table entries of request r's keys, from its first key on.
__device__ __forceinline__ const int32_t* req_bt(const FwdParams& p, int r) {
    if (p.casc_len > 0) return r == 0 ? p.bt : p.bt + (int64_t)(r - 1) * p.bt_stride + p.casc_len / p.bs;
    return p.bt + (int64_t)r * p.bt_stride;
}
// Whether request r's keys take the causal mask.
__device__ __forceinline__ bool req_causal(const FwdParams& p, int r) {
    return p.causal && !(p.casc_len > 0 && r == 0);
}

enum class KvType { BF16, FP8, F32 };

// Bytes of the device-resident scratch array behind pkv_varlen_fwd_noalloc
// (one per GPU, held until the process ends), and its device address on the
// current device (looked up on the first call per device).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_for_current_device(void** ptr);

// Launchers return hipSuccess or the launch error.
hipError_t launch_decode(const FwdParams& p, KvType kv, hipStream_t s);
hipError_t launch_decode_balanced(const FwdParams& p, KvType kv, hipStream_t s);
hipError_t launch_combine_balanced(const FwdParams& p, hipStream_t s);
hipError_t launch_combine_cascade(const FwdParams& p, hipStream_t s);
hipError_t launch_prefill(const FwdParams& p, KvType kv, bool q8, hipStream_t s);
hipError_t launch_generic(const FwdParams& p, KvType kv, bool q_f32, hipStream_t s);
hipError_t launch_combine(const FwdParams& p, bool out_f32, hipStream_t s);
hipError_t launch_merge(void* out, float* out_lse, const void* po, const float* plse, const void* so,
                        const float* slse, int64_t T, int32_t H, int32_t hd, bool f32, hipStream_t s);
hipError_t launch_cache_write(const void* key, const void* value, int src_f32, void* kc, void* vc, int cache_kind,
                              const int64_t* slots, int64_t T, int32_t Hkv, int32_t hd, const float* ks,
                              const float* vs, hipStream_t s);

// Decode kernel geometry: rows (q tokens x heads of a group) per work item,
// keys per tile, waves per workgroup.
constexpr int kDecodeRows = 16;
constexpr int kDecodeTile = 32;
constexpr int kDecodeWaves = 4;
// Balanced decode: waves in the grid for a bf16 cache (one workgroup of 4
// waves on each of the 256 CUs of MI355X; twice as many waves, all resident,
// stream the paged KV slightly slower, so the memory system is past
// saturation there; fp8 caches use twice as many) and the largest batch whose
// schedule each wave derives by itself.
constexpr int kBalancedWaves = 1024;
// Balanced decode items hold up to kDecodeMaxRows query rows (q_len x group)
// as blocks of 16, for head sizes up to kDecodeMaxRbHead (larger heads: 16).
// (Four blocks fit the register file of a lone wave at head size 128, but
// their tile computation no longer hides under the tile loads and their
// partial states cost a tenth of the KV bytes again: the prefill kernel
// serves such items faster.)
constexpr int kDecodeMaxRows = 32;
constexpr int kDecodeMaxRbHead = 128;
constexpr int kBalancedMaxSeqs = 1024;
// Accelerator complex dies of MI355X; consecutive workgroup ids go to
// consecutive XCDs, each with its own L2.
constexpr int kXcds = 8;
// Prefill kernel geometry: four waves of 32 query rows per workgroup sharing
// K/V tiles of 64 keys in LDS (two workgroups per CU up to head size 128).
constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillWaves = 4;
// Query rows per work item of the prefill kernel's key-split mode (two waves
// per 32 rows, each on half of every tile), taken when no item of a paged
// batch has more rows than this.
constexpr int kPrefillSplitRows = 64;
constexpr int prefill_tile(int) { return 64; }
constexpr int prefill_rows(int) { return kPrefillRowsPerWave * kPrefillWaves; }
// The largest GQA group the prefill kernel packs (query rows per workgroup).
constexpr int kPrefillMaxGroup = kPrefillRowsPerWave * kPrefillWaves;

}  // namespace pkv
