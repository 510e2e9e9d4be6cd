// pkv_api.cpp -- host side of the C ABI declared in include/pkvflash.h:
// argument validation, the choice of kernel and of the KV split, launches on
// the caller's stream, error reporting and optional kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/pkvflash.h"
#include "pkv_kernels.h"

using namespace pkv;

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pkv_status fail(pkv_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

pkv_status ok() {
    g_err.clear();
    return PKV_OK;
}

pkv_status hip_fail(hipError_t e, const char* what) {
    return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

enum class Kind { Decode, DecodeBalanced, Prefill, Generic };

struct Plan {
    Kind kind;
    int32_t splits;
    int32_t split_len;
    int32_t n_qtiles;
    int32_t dec_rows;  // balanced decode: query rows per item slot
    bool pf_ksplit;    // prefill: key-split items of kPrefillSplitRows rows
    size_t workspace;  // bytes needed for `splits`
};

// Decode with a sliding window of at most this many keys, over at least this
// many (request, kv head) items, takes the unsplit decode grid (make_plan).
constexpr int kWindowPerItem = 1024;
constexpr int kWindowMinItems = 256;

// Query rows per balanced-decode item slot (16-row blocks) for items of
// `rows` rows, or 0 when the balanced kernel does not take them: up to 32
// rows over a paged cache with head size up to 128, else up to 16.
int32_t decode_rows(const pkv_varlen_args* a, int64_t rows) {
    if (rows <= kDecodeRows) return kDecodeRows;
    if (a->block_table == nullptr || a->head_size > kDecodeMaxRbHead || rows > kDecodeMaxRows) return 0;
    return 2 * kDecodeRows;
}

bool mfma_head(int hd) { return hd == 64 || hd == 128 || hd == 256; }

// Sizes, types and their consistency (no pointer checks).
pkv_status validate_sizes(const pkv_varlen_args* a);

// Everything pkv_varlen_fwd needs: sizes plus the required pointers.
pkv_status validate(const pkv_varlen_args* a) {
    pkv_status st = validate_sizes(a);
    if (st != PKV_OK || a->num_tokens == 0) return st;
    if (!a->q || !a->k_cache || !a->v_cache || !a->out || !a->query_start_loc)
        return fail(PKV_ERR_INVALID_ARG, "q, k_cache, v_cache, out and query_start_loc must be non-NULL");
    if (a->block_table && !a->seq_lens) return fail(PKV_ERR_INVALID_ARG, "a paged cache needs seq_lens");
    if (a->kv_dtype == PKV_FP8_E4M3FN && (!a->k_scale || !a->v_scale))
        return fail(PKV_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
    if (a->q_dtype == PKV_FP8_E4M3FN && !a->q_scale) return fail(PKV_ERR_INVALID_ARG, "an fp8 q needs q_scale");
    return ok();
}

pkv_status validate_sizes(const pkv_varlen_args* a) {
    if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
    if (a->num_tokens < 0 || a->num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "negative num_tokens or num_seqs");
    if (a->num_tokens >= (int64_t(1) << 31)) return fail(PKV_ERR_UNSUPPORTED, "num_tokens must be < 2^31");
    if (a->num_tokens > 0 && a->num_seqs == 0) return fail(PKV_ERR_INVALID_ARG, "tokens without sequences");
    if (a->num_heads <= 0 || a->num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_heads and num_kv_heads must be positive");
    if (a->num_heads % a->num_kv_heads != 0)
        return fail(PKV_ERR_INVALID_ARG, "num_heads (%d) is not a multiple of num_kv_heads (%d)", a->num_heads, a->num_kv_heads);
    if (a->num_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_heads must be <= 65535");
    if (a->head_size <= 0 || a->head_size % 8 != 0 || a->head_size > 256)
        return fail(PKV_ERR_UNSUPPORTED, "head_size %d: must be a multiple of 8 and at most 256", a->head_size);
    const bool ok_types = (a->q_dtype == PKV_BF16 && (a->kv_dtype == PKV_BF16 || a->kv_dtype == PKV_FP8_E4M3FN)) ||
                          (a->q_dtype == PKV_F32 && a->kv_dtype == PKV_F32) ||
                          (a->q_dtype == PKV_FP8_E4M3FN && a->kv_dtype == PKV_FP8_E4M3FN);
    if (!ok_types) return fail(PKV_ERR_UNSUPPORTED, "unsupported (q_dtype, kv_dtype) = (%d, %d)", a->q_dtype, a->kv_dtype);
    if (a->q_dtype == PKV_FP8_E4M3FN && (a->head_size != 128 || a->num_heads / a->num_kv_heads > kPrefillMaxGroup))
        return fail(PKV_ERR_UNSUPPORTED, "an fp8 q needs head_size 128 and a group of at most %d heads",
                    kPrefillMaxGroup);
    if (!std::isfinite(a->softmax_scale) || !(a->softmax_scale > 0.f))
        return fail(PKV_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
    if (a->sliding_window < 0) return fail(PKV_ERR_INVALID_ARG, "sliding_window must be >= 0 (0: no window)");
    if (!(a->softcap >= 0.f) || !std::isfinite(a->softcap))
        return fail(PKV_ERR_INVALID_ARG, "softcap must be finite and >= 0 (0: off)");
    if (a->num_splits < 0 || a->num_splits > 256) return fail(PKV_ERR_INVALID_ARG, "num_splits must be in [0, 256]");
    if (a->num_tokens == 0) return ok();
    if (a->num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_seqs must be <= 65535");
    if (a->max_seqlen_q <= 0) return fail(PKV_ERR_INVALID_ARG, "max_seqlen_q must be positive");
    if (a->num_tokens > (int64_t)a->num_seqs * a->max_seqlen_q)
        return fail(PKV_ERR_INVALID_ARG, "num_tokens exceeds num_seqs * max_seqlen_q");
    if (a->block_table) {
        if (a->block_size <= 0) return fail(PKV_ERR_INVALID_ARG, "block_size must be positive");
        if (a->num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
        if (a->num_blocks * (int64_t)a->block_size >= (int64_t(1) << 31))
            return fail(PKV_ERR_UNSUPPORTED, "num_blocks * block_size must be < 2^31");
        // (causal: every request's KV includes its own new tokens; a
        // non-causal pass, such as a cascade's prefix pass, may have more
        // queries than keys)
        if (a->causal && a->max_seqlen_k < a->max_seqlen_q)
            return fail(PKV_ERR_INVALID_ARG, "max_seqlen_k (%d) < max_seqlen_q (%d): seq_lens include the new tokens",
                        a->max_seqlen_k, a->max_seqlen_q);
        if (a->max_seqlen_k < 0) return fail(PKV_ERR_INVALID_ARG, "max_seqlen_k must be >= 0");
        if (a->block_table_stride < cdiv(a->max_seqlen_k, a->block_size))
            return fail(PKV_ERR_INVALID_ARG, "block_table_stride %lld < ceil(max_seqlen_k / block_size) = %lld",
                        (long long)a->block_table_stride, (long long)cdiv(a->max_seqlen_k, a->block_size));
    }
    return ok();
}

// Waves of the balanced decode grid: one workgroup per CU for bf16 caches;
// fp8 tiles carry half the bytes, so two workgroups per CU keep as many bytes
// in flight (where their LDS and registers fit: head size up to 128, items of
// one 16-row block).
static int64_t balanced_waves(const pkv_varlen_args* a, int32_t dec_rows) {
    return a->kv_dtype == PKV_FP8_E4M3FN && a->head_size <= 128 && dec_rows == kDecodeRows ? 2 * kBalancedWaves
                                                                                           : kBalancedWaves;
}

// balanced_ok false: plan without the balanced decode schedule (no room for
// its partials).
Plan make_plan(const pkv_varlen_args* a, bool balanced_ok = true) {
    Plan pl{};
    const int g = a->num_heads / a->num_kv_heads;
    const bool paged = a->block_table != nullptr;
    int64_t max_k = paged ? a->max_seqlen_k : a->max_seqlen_q;
    // With a sliding window a request's keys start at its window base (the
    // window start of its first query token, rounded down to 64 keys), so
    // the splits only need to cover the span from there to its last key.
    if (a->sliding_window > 0)
        max_k = std::min<int64_t>(max_k, (int64_t)a->sliding_window - 1 + a->max_seqlen_q + 63);
    const bool q8 = a->q_dtype == PKV_FP8_E4M3FN;  // fp8 QK^T: the prefill kernel, whatever the shape
    const bool mfma = (a->q_dtype == PKV_BF16 || q8) && mfma_head(a->head_size) && g <= kPrefillMaxGroup;
    int64_t items;
    int align;
    const int32_t drows = decode_rows(a, (int64_t)a->max_seqlen_q * g);
    // With a short sliding window no request costs more than the window, and
    // every request longer than it costs the same, so the plain decode grid
    // (one workgroup per request and kv head, unsplit) is balanced by itself
    // and needs no merge: measured faster than the balanced schedule on 64
    // requests for every window from 128 to 2048 keys. The rule stops at
    // kWindowPerItem keys, where a batch of one long and many short requests
    // still costs at most a few tile rounds more than the balanced schedule,
    // and needs enough items to give every CU a workgroup.
    const bool short_window = a->sliding_window > 0 && a->sliding_window <= kWindowPerItem &&
                              a->num_splits == 0 && (int64_t)a->max_seqlen_q * g <= kDecodeRows &&
                              (int64_t)a->num_seqs * a->num_kv_heads >= kWindowMinItems;
    if (balanced_ok && !short_window && mfma && !q8 && drows > 0 && a->num_splits == 0 &&
        a->num_seqs <= kBalancedMaxSeqs) {
        // balanced decode: balanced_waves() waves share the KV tiles equally
        pl.kind = Kind::DecodeBalanced;
        pl.dec_rows = drows;
        pl.splits = (int32_t)balanced_waves(a, drows);
        pl.split_len = kDecodeTile;
        const int64_t slots = pl.splits + (int64_t)a->num_seqs * a->num_kv_heads;
        pl.workspace = (size_t)slots * drows * (a->head_size + 1) * sizeof(float) +
                       (size_t)(a->num_seqs + 1) * sizeof(int32_t);
        return pl;
    }
    if (mfma && !q8 && (int64_t)a->max_seqlen_q * g <= kDecodeRows) {
        pl.kind = Kind::Decode;
        items = (int64_t)a->num_seqs * a->num_kv_heads;
        align = kDecodeTile * kDecodeWaves;
    } else if (mfma) {
        pl.kind = Kind::Prefill;
        // key-split items of 64 rows when no request's rows need more (a
        // paged cache, bf16 q, head size up to 128)
        pl.pf_ksplit = g <= kPrefillSplitRows && (int64_t)a->max_seqlen_q * g <= kPrefillSplitRows && paged && !q8 &&
                       a->head_size <= 128;
        const int tpw = (pl.pf_ksplit ? kPrefillSplitRows : prefill_rows(a->head_size)) / g;
        pl.n_qtiles = (int32_t)cdiv(a->max_seqlen_q, tpw);
        items = (int64_t)a->num_seqs * a->num_kv_heads * pl.n_qtiles;
        align = prefill_tile(a->head_size) * 4;
    } else {
        pl.kind = Kind::Generic;
        items = a->num_tokens * a->num_heads;
        align = 64;
    }
    int64_t S = 1;
    if (a->num_splits > 1) {
        S = a->num_splits;
    } else if (a->num_splits == 0 && pl.kind != Kind::Generic && !(short_window && pl.kind == Kind::Decode)) {
        // Split only when there are too few work items to occupy 256 CUs, and
        // keep at least 512 keys of work per split. (Prefill partials are
        // written for every query row, so splitting a prefill that already
        // fills the chip costs far more traffic than it saves.)
        const int64_t by_len = cdiv(max_k, 512);
        const int64_t enough = pl.kind == Kind::Prefill ? 256 : 2048;
        if (items < enough) S = std::min<int64_t>(by_len, std::max<int64_t>(1, cdiv(2 * enough, items)));
        S = std::max<int64_t>(1, std::min<int64_t>(S, 64));
    }
    if (S > 1) {
        int64_t len = cdiv(cdiv(max_k, S), align) * align;
        if (len <= 0) len = align;
        S = cdiv(max_k, len);
        pl.split_len = (int32_t)len;
    }
    if (S <= 1) {
        S = 1;
        pl.split_len = (int32_t)std::max<int64_t>(max_k, 1);
    }
    pl.splits = (int32_t)S;
    pl.workspace = S > 1 ? (size_t)S * a->num_tokens * a->num_heads * (a->head_size + 1) * sizeof(float) : 0;
    return pl;
}

// ------------------------------------------------------------------ timing

struct Timing {
    bool on = false;
    std::vector<hipEvent_t> ev;  // 4 per call: main start/end, merge start/end
    std::vector<char> has_merge;
    int calls = 0;
};
Timing g_tim;
constexpr int kTimingCap = 4096;

}  // namespace

extern "C" {

size_t pkv_varlen_args_size(void) { return sizeof(pkv_varlen_args); }

pkv_status pkv_varlen_check(const pkv_varlen_args* a) { return validate(a); }

int32_t pkv_varlen_num_splits(const pkv_varlen_args* a) {
    if (validate_sizes(a) != PKV_OK) return 0;
    return make_plan(a).splits;
}

size_t pkv_varlen_workspace_size(const pkv_varlen_args* a) {
    if (validate_sizes(a) != PKV_OK) return 0;
    return make_plan(a).workspace;
}

}  // extern "C"

namespace {

// How one forward pass reads the batch's metadata (cascade passes; the
// defaults are a plain forward).
struct PassOpts {
    int32_t single_len = 0;  // > 0: all tokens form one request with this KV length
    int32_t seq_off = 0;     // keys before this index are another pass's
    int32_t casc_len = 0;    // > 0: both cascade passes as one balanced decode (request 0 of
                             // a->num_seqs is the shared prefix of this many keys)
};

// One forward over validated arguments (a->workspace holds the partials).
pkv_status run_fwd(const pkv_varlen_args* a, const PassOpts& o, hipStream_t s) {
    Plan pl = make_plan(a);
    if (o.casc_len > 0 && (pl.kind != Kind::DecodeBalanced || a->workspace == nullptr ||
                           a->workspace_bytes < pl.workspace))
        return fail(PKV_ERR_WORKSPACE, "the one-launch cascade needs the balanced decode and %zu workspace bytes",
                    pl.workspace);
    if (pl.kind == Kind::DecodeBalanced && (a->workspace == nullptr || a->workspace_bytes < pl.workspace)) {
        // no room for the balanced schedule's partials: the other kernels,
        // unsplit unless their partials fit
        pl = make_plan(a, false);
    }
    if (pl.kind != Kind::DecodeBalanced && pl.splits > 1 &&
        (a->workspace == nullptr || a->workspace_bytes < pl.workspace)) {
        if (a->num_splits > 1)
            return fail(PKV_ERR_WORKSPACE, "num_splits=%d needs %zu workspace bytes, got %zu", pl.splits, pl.workspace,
                        a->workspace ? a->workspace_bytes : (size_t)0);
        // automatic choice without room for partials: run unsplit
        pl.splits = 1;
        pl.split_len = (int32_t)std::max<int64_t>(a->block_table ? a->max_seqlen_k : a->max_seqlen_q, 1);
        pl.workspace = 0;
    }
    FwdParams p{};
    p.q = a->q;
    p.k_cache = a->k_cache;
    p.v_cache = a->v_cache;
    p.out = a->out;
    p.lse = a->lse;
    p.qsl = a->query_start_loc;
    p.seq_lens = a->block_table ? a->seq_lens : nullptr;
    p.bt = a->block_table;
    p.k_scale = a->k_scale;
    p.v_scale = a->v_scale;
    p.q_scale = a->q_scale;
    p.bt_stride = a->block_table_stride;
    p.T = a->num_tokens;
    p.B = a->num_seqs;
    p.H = a->num_heads;
    p.Hkv = a->num_kv_heads;
    p.g = a->num_heads / a->num_kv_heads;
    p.hd = a->head_size;
    p.bs = a->block_table ? a->block_size : 1;
    p.bs_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == p.bs) p.bs_shift = sh;
    p.num_splits = pl.splits;
    p.split_len = pl.split_len;
    p.n_qtiles = pl.n_qtiles;
    p.pf_ksplit = pl.kind == Kind::Prefill && pl.pf_ksplit ? 1 : 0;
    p.causal = a->causal ? 1 : 0;
    p.scale_log2 = a->softmax_scale * 1.4426950408889634f;  // log2(e): kernels use exp2
    p.window_left = a->sliding_window - 1;  // -1: none
    p.softcap_l2 = a->softcap > 0.f ? a->softcap * 1.4426950408889634f : 0.f;
    p.softcap_inv2 = a->softcap > 0.f ? 2.f / a->softcap : 0.f;
    p.sinks = a->sinks;
    p.alibi = a->alibi_slopes;
    p.single_len = o.single_len;
    p.seq_off = o.seq_off;
    p.casc_len = o.casc_len;
    if (pl.kind == Kind::DecodeBalanced) {
        const int64_t slots = pl.splits + (int64_t)a->num_seqs * a->num_kv_heads;
        p.sk_waves = pl.splits;
        p.dec_rows = pl.dec_rows;
        // (no item has more rows than the longest request's tokens x the group)
        p.merge_rows = (int32_t)std::min<int64_t>(pl.dec_rows, ((int64_t)a->max_seqlen_q * p.g + 7) / 8 * 8);
        p.part_o = (float*)a->workspace;
        p.part_lse = p.part_o + (size_t)slots * pl.dec_rows * a->head_size;
        p.sk_prefix = (int32_t*)(p.part_lse + (size_t)slots * pl.dec_rows);
    } else if (pl.splits > 1) {
        p.part_o = (float*)a->workspace;
        p.part_lse = p.part_o + (size_t)pl.splits * a->num_tokens * a->num_heads * a->head_size;
    }
    const KvType kv = a->kv_dtype == PKV_FP8_E4M3FN ? KvType::FP8 : a->kv_dtype == PKV_F32 ? KvType::F32 : KvType::BF16;

    const bool timed = g_tim.on && g_tim.calls < kTimingCap;
    hipEvent_t* ev = timed ? &g_tim.ev[4 * g_tim.calls] : nullptr;
    if (timed) {
        hipError_t e = hipEventRecord(ev[0], s);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    hipError_t e;
    switch (pl.kind) {
        case Kind::DecodeBalanced: e = launch_decode_balanced(p, kv, s); break;
        case Kind::Decode: e = launch_decode(p, kv, s); break;
        case Kind::Prefill: e = launch_prefill(p, kv, a->q_dtype == PKV_FP8_E4M3FN, s); break;
        default: e = launch_generic(p, kv, a->q_dtype == PKV_F32, s); break;
    }
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    if (timed) {
        e = hipEventRecord(ev[1], s);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    const bool merge = pl.kind == Kind::DecodeBalanced || pl.splits > 1;
    if (merge) {
        if (timed) (void)hipEventRecord(ev[2], s);
        e = pl.kind != Kind::DecodeBalanced ? launch_combine(p, a->q_dtype == PKV_F32, s)
            : o.casc_len > 0              ? launch_combine_cascade(p, s)
                                          : launch_combine_balanced(p, s);
        if (e != hipSuccess) return hip_fail(e, "split merge kernel launch");
        if (timed) (void)hipEventRecord(ev[3], s);
    }
    if (timed) {
        g_tim.has_merge[g_tim.calls] = merge;
        ++g_tim.calls;
    }
    return ok();
}

// ------------------------------------------------------------------ cascade

// Round up to 256 bytes (each workspace region starts aligned).
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The two passes of a cascade over the batch `a` with a shared prefix of P
// keys, and where their results go in the workspace:
// [prefix out][prefix lse][suffix out][suffix lse][the passes' own partials].
struct Cascade {
    pkv_varlen_args pre, suf;
    PassOpts pre_o, suf_o;
    size_t o_bytes, l_bytes, pass_ws, total;
    // one launch: the batch as a balanced decode with the shared prefix as
    // request 0 (every token of the batch against it, no causal mask)
    bool fused;
    pkv_varlen_args one;
    PassOpts one_o;
};

// Whether a cascade runs as one balanced decode launch: `one` is the batch
// with the prefix pass as a further request of every token (num_seqs + 1,
// max_seqlen_q = num_tokens).
bool one_launch_cascade(const pkv_varlen_args& one) {
    if (one.num_splits != 0) return false;
    const std::string err = g_err;  // (a failed check here is no error of the caller's)
    const bool valid = validate_sizes(&one) == PKV_OK;
    g_err = err;
    return valid && make_plan(&one).kind == Kind::DecodeBalanced;
}

pkv_status cascade_plan(const pkv_varlen_args* a, int32_t P, Cascade& c) {
    if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
    if (!a->block_table) return fail(PKV_ERR_INVALID_ARG, "a cascade needs a paged cache (block_table)");
    if (a->alibi_slopes)
        return fail(PKV_ERR_UNSUPPORTED, "ALiBi needs each query's own position, which the prefix pass does not keep");
    if (a->sliding_window > 0) return fail(PKV_ERR_UNSUPPORTED, "a cascade with a sliding window is not supported");
    if (a->block_size <= 0 || P <= 0 || P % a->block_size != 0)
        return fail(PKV_ERR_INVALID_ARG, "common_prefix_len %d must be a positive multiple of block_size %d", P,
                    a->block_size);
    if (P > a->max_seqlen_k)
        return fail(PKV_ERR_INVALID_ARG, "common_prefix_len %d > max_seqlen_k %d", P, a->max_seqlen_k);
    const int T = (int)a->num_tokens;
    // prefix pass: every token against the P shared keys (the first row of
    // the block table), as one request, not causal
    c.pre = *a;
    c.pre.num_seqs = 1;
    c.pre.max_seqlen_q = T;
    c.pre.max_seqlen_k = P;
    c.pre.causal = 0;
    c.pre.sinks = nullptr;  // the sink joins the suffix pass only
    c.pre_o = PassOpts{};
    c.pre_o.single_len = P;
    // suffix pass: each request against its own keys past the prefix, with
    // the block table from the first page after it
    c.suf = *a;
    c.suf.block_table = a->block_table + P / a->block_size;
    c.suf.max_seqlen_k = a->max_seqlen_k - P;
    c.suf_o = PassOpts{};
    c.suf_o.seq_off = P;
    pkv_status st = validate_sizes(&c.pre);
    if (st != PKV_OK) return st;
    st = validate_sizes(&c.suf);
    if (st != PKV_OK) return st;
    const size_t out_elt = a->q_dtype == PKV_F32 ? 4 : 2;
    c.o_bytes = align256((size_t)a->num_tokens * a->num_heads * a->head_size * out_elt);
    c.l_bytes = align256((size_t)a->num_tokens * a->num_heads * sizeof(float));
    c.pass_ws = std::max(make_plan(&c.pre).workspace, make_plan(&c.suf).workspace);
    c.total = 2 * (c.o_bytes + c.l_bytes) + c.pass_ws;
    // The one-launch form, when the batch is decode-shaped: all of its query
    // rows (every token x the group) fit one item of the balanced decode.
    c.one = *a;
    c.one.num_seqs = a->num_seqs + 1;
    c.one.max_seqlen_q = T;
    c.one_o = PassOpts{};
    c.one_o.casc_len = P;
    c.fused = one_launch_cascade(c.one);
    if (c.fused) c.total = make_plan(&c.one).workspace;
    return ok();
}

}  // namespace

extern "C" {

pkv_status pkv_varlen_fwd(const pkv_varlen_args* a, void* stream) {
    pkv_status st = validate(a);
    if (st != PKV_OK || a->num_tokens == 0) return st;
    return run_fwd(a, PassOpts{}, (hipStream_t)stream);
}

pkv_status pkv_varlen_fwd_noalloc(const pkv_varlen_args* a, void* stream) {
    pkv_status st = validate(a);
    if (st != PKV_OK || a->num_tokens == 0) return st;
    // the plan is the one pkv_varlen_fwd makes; its partials must fit the scratch
    const size_t need = make_plan(a).workspace;
    if (need > kScratchBytes)
        return fail(PKV_ERR_WORKSPACE,
                    "this forward needs %zu bytes of split-KV scratch; the static scratch holds %zu "
                    "(num_splits = 1 needs none)", need, kScratchBytes);
    void* ptr = nullptr;
    hipError_t e = scratch_for_current_device(&ptr);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    pkv_varlen_args b = *a;
    b.workspace = ptr;
    b.workspace_bytes = kScratchBytes;
    return run_fwd(&b, PassOpts{}, (hipStream_t)stream);
}

size_t pkv_cascade_workspace_size(const pkv_varlen_args* a, int32_t common_prefix_len) {
    if (validate_sizes(a) != PKV_OK || a->num_tokens == 0) return 0;
    Cascade c;
    if (cascade_plan(a, common_prefix_len, c) != PKV_OK) return 0;
    return c.total;
}

pkv_status pkv_cascade_fwd(const pkv_varlen_args* a, int32_t common_prefix_len, void* stream) {
    pkv_status st = validate(a);
    if (st != PKV_OK || a->num_tokens == 0) return st;
    Cascade c;
    st = cascade_plan(a, common_prefix_len, c);
    if (st != PKV_OK) return st;
    if (!a->workspace || a->workspace_bytes < c.total)
        return fail(PKV_ERR_WORKSPACE, "a cascade needs %zu workspace bytes, got %zu", c.total,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (c.fused) {  // both passes and the merge: one decode launch, one merge launch
        c.one.workspace = a->workspace;
        c.one.workspace_bytes = a->workspace_bytes;
        return run_fwd(&c.one, c.one_o, (hipStream_t)stream);
    }
    uint8_t* ws = (uint8_t*)a->workspace;
    void* o_p = ws;
    float* l_p = (float*)(ws + c.o_bytes);
    void* o_s = ws + c.o_bytes + c.l_bytes;
    float* l_s = (float*)(ws + 2 * c.o_bytes + c.l_bytes);
    void* pass_ws = ws + 2 * (c.o_bytes + c.l_bytes);
    hipStream_t s = (hipStream_t)stream;
    c.pre.out = o_p;
    c.pre.lse = l_p;
    c.pre.workspace = pass_ws;
    c.pre.workspace_bytes = c.pass_ws;
    st = run_fwd(&c.pre, c.pre_o, s);
    if (st != PKV_OK) return st;
    c.suf.out = o_s;
    c.suf.lse = l_s;
    c.suf.workspace = pass_ws;
    c.suf.workspace_bytes = c.pass_ws;
    st = run_fwd(&c.suf, c.suf_o, s);
    if (st != PKV_OK) return st;
    const bool f32 = a->q_dtype == PKV_F32;
    hipError_t e = launch_merge(a->out, a->lse, o_p, l_p, o_s, l_s, a->num_tokens, a->num_heads, a->head_size, f32, s);
    if (e != hipSuccess) return hip_fail(e, "cascade merge launch");
    return ok();
}

pkv_status pkv_cache_write(const void* key, const void* value, pkv_dtype src_dtype, void* k_cache, void* v_cache,
                           pkv_dtype cache_dtype, const int64_t* slot_mapping, int64_t num_tokens,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size, int64_t num_blocks,
                           const float* k_scale, const float* v_scale, void* stream) {
    if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_kv_heads <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_INVALID_ARG, "num_kv_heads, block_size and num_blocks must be positive");
    if (head_size <= 0 || head_size % 8 != 0 || head_size > 256)
        return fail(PKV_ERR_UNSUPPORTED, "head_size %d: must be a multiple of 8 and at most 256", head_size);
    int kind;
    if (src_dtype == cache_dtype && (src_dtype == PKV_F32 || src_dtype == PKV_BF16)) kind = 0;
    else if (src_dtype == PKV_F32 && cache_dtype == PKV_BF16) kind = 1;
    else if ((src_dtype == PKV_F32 || src_dtype == PKV_BF16) && cache_dtype == PKV_FP8_E4M3FN) kind = 2;
    else return fail(PKV_ERR_UNSUPPORTED, "unsupported (src_dtype, cache_dtype) = (%d, %d)", src_dtype, cache_dtype);
    if (kind == 2 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
    if (num_tokens == 0) return ok();
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_ERR_INVALID_ARG, "key, value, k_cache, v_cache and slot_mapping must be non-NULL");
    if (2 * num_tokens * ((int64_t)num_kv_heads * head_size / 8) >= (int64_t(1) << 31) * 256)
        return fail(PKV_ERR_UNSUPPORTED, "too many tokens for one launch");
    hipError_t e = launch_cache_write(key, value, src_dtype == PKV_F32, k_cache, v_cache, kind, slot_mapping,
                                      num_tokens, num_kv_heads, head_size, k_scale, v_scale, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "cache write launch");
    return ok();
}

pkv_status pkv_merge_attn_states(void* out, float* out_lse, const void* prefix_out, const float* prefix_lse,
                                 const void* suffix_out, const float* suffix_lse, int64_t num_tokens,
                                 int32_t num_heads, int32_t head_size, pkv_dtype dtype, void* stream) {
    if (num_tokens < 0 || num_heads <= 0 || head_size <= 0)
        return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0, num_heads and head_size positive");
    if (head_size % 8 != 0 || head_size > 256)
        return fail(PKV_ERR_UNSUPPORTED, "head_size %d: must be a multiple of 8 and at most 256", head_size);
    if (dtype != PKV_BF16 && dtype != PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "merge supports BF16 and F32 states");
    if (num_tokens == 0) return ok();
    if (!out || !prefix_out || !prefix_lse || !suffix_out || !suffix_lse)
        return fail(PKV_ERR_INVALID_ARG, "out, prefix_out, prefix_lse, suffix_out and suffix_lse must be non-NULL");
    if (num_tokens * num_heads * (head_size / 4) >= (int64_t(1) << 31) * 256)
        return fail(PKV_ERR_UNSUPPORTED, "too many rows for one launch");
    hipError_t e = launch_merge(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse, num_tokens, num_heads,
                                head_size, dtype == PKV_F32, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return ok();
}

pkv_status pkv_cascade_choose(int32_t common_prefix_len, int32_t num_seqs, const int32_t* host_seq_lens,
                              int64_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                              pkv_dtype kv_dtype, int32_t sliding_window, int32_t* use_cascade, double* t_plain_us,
                              double* t_cascade_us) {
    // Read rates (bytes per us) and fixed costs of the plain decode and the
    // two cascade forms, and the share of the plain form's prefix re-reads
    // that reach HBM as a ramp in the prefix's part of the mean KV length;
    // all fitted to measurements on MI355X (24 shared-prefix decode batches,
    // the cascade forms by least squares, the ramp by the time a wrong choice
    // costs)
    constexpr double kPlainRate = 5.6e6, kPlainFixedUs = 17.0;
    constexpr double kOneRate = 5.8e6, kOneFixedUs = 32.0;
    constexpr double kThreeRate = 5.5e6, kThreeFixedUs = 40.0;
    constexpr double kMissFrom = 0.2, kMissSlope = 2.4, kMissMax = 0.6;
    constexpr int32_t kMinPrefix = 256;
    if (!use_cascade || num_seqs < 0 || (num_seqs > 0 && !host_seq_lens) || num_tokens < 0 || num_heads <= 0 ||
        num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || head_size <= 0 || common_prefix_len < 0 ||
        sliding_window < 0)
        return fail(PKV_ERR_INVALID_ARG, "invalid cascade query");
    if (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3FN && kv_dtype != PKV_F32)
        return fail(PKV_ERR_UNSUPPORTED, "unknown kv_dtype %d", (int)kv_dtype);
    const double per_key = 2.0 * num_kv_heads * head_size * (kv_dtype == PKV_FP8_E4M3FN ? 1 : kv_dtype == PKV_F32 ? 4 : 2);
    int64_t keys = 0;
    bool prefix_fits = num_seqs > 0;
    for (int32_t r = 0; r < num_seqs; ++r) {
        if (host_seq_lens[r] < 0) return fail(PKV_ERR_INVALID_ARG, "negative seq_lens[%d]", r);
        keys += host_seq_lens[r];
        prefix_fits = prefix_fits && host_seq_lens[r] > common_prefix_len;  // every request keeps a suffix
    }
    const int64_t rereads = prefix_fits ? (int64_t)(num_seqs - 1) * common_prefix_len : 0;
    const int64_t unique = keys - rereads;
    const double f = keys > 0 ? (double)common_prefix_len * num_seqs / (double)keys : 0.0;
    const double miss = std::min(kMissMax, std::max(0.0, kMissSlope * (f - kMissFrom)));
    const double tp = kPlainFixedUs + (unique + miss * rereads) * per_key / kPlainRate;
    // the batch as pkv_cascade_fwd would see it (a bf16 q; the table itself
    // is never read here)
    pkv_varlen_args one{};
    int32_t max_len = 0;
    for (int32_t r = 0; r < num_seqs; ++r) max_len = std::max(max_len, host_seq_lens[r]);
    one.num_tokens = num_tokens;
    one.num_seqs = num_seqs + 1;
    one.num_heads = num_heads;
    one.num_kv_heads = num_kv_heads;
    one.head_size = head_size;
    one.q_dtype = kv_dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
    one.kv_dtype = kv_dtype;
    one.softmax_scale = 1.f;
    one.causal = 1;
    one.max_seqlen_q = (int32_t)std::min<int64_t>(std::max<int64_t>(num_tokens, 1), INT32_MAX);
    one.max_seqlen_k = std::max(max_len, one.max_seqlen_q);
    one.block_table = &max_len;  // (any non-NULL address: a paged batch)
    one.block_size = 16;
    one.num_blocks = 1;
    one.block_table_stride = cdiv(one.max_seqlen_k, one.block_size);
    const bool one_launch = num_tokens > 0 && one_launch_cascade(one);
    const double tc = one_launch ? kOneFixedUs + unique * per_key / kOneRate
                                 : kThreeFixedUs + unique * per_key / kThreeRate;
    if (t_plain_us) *t_plain_us = tp;
    if (t_cascade_us) *t_cascade_us = tc;
    *use_cascade = common_prefix_len >= kMinPrefix && sliding_window == 0 && prefix_fits && tc < tp ? 1 : 0;
    return ok();
}

const char* pkv_last_error(void) { return g_err.c_str(); }

int32_t pkv_version(void) { return 100; }

pkv_status pkv_timing_enable(int32_t on) {
    if (on && !g_tim.on) {
        g_tim.ev.assign(4 * kTimingCap, nullptr);
        g_tim.has_merge.assign(kTimingCap, 0);
        for (auto& e : g_tim.ev) {
            hipError_t r = hipEventCreate(&e);
            if (r != hipSuccess) return hip_fail(r, "hipEventCreate");
        }
        g_tim.calls = 0;
        g_tim.on = true;
    } else if (!on && g_tim.on) {
        for (auto& e : g_tim.ev)
            if (e) (void)hipEventDestroy(e);
        g_tim.ev.clear();
        g_tim.has_merge.clear();
        g_tim.calls = 0;
        g_tim.on = false;
    }
    return ok();
}

// Milliseconds of call i's main kernel and merge kernel (0 without one).
static pkv_status timing_of(int i, float& main_ms, float& merge_ms) {
    hipError_t e = hipEventSynchronize(g_tim.ev[4 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    e = hipEventElapsedTime(&main_ms, g_tim.ev[4 * i], g_tim.ev[4 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    merge_ms = 0.f;
    if (g_tim.has_merge[i]) {
        e = hipEventSynchronize(g_tim.ev[4 * i + 3]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        e = hipEventElapsedTime(&merge_ms, g_tim.ev[4 * i + 2], g_tim.ev[4 * i + 3]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    }
    return ok();
}

pkv_status pkv_timing_collect(int32_t* calls, double* main_ms, double* merge_ms) {
    double a = 0, b = 0;
    for (int i = 0; i < g_tim.calls; ++i) {
        float m = 0.f, g = 0.f;
        pkv_status st = timing_of(i, m, g);
        if (st != PKV_OK) return st;
        a += m;
        b += g;
    }
    if (calls) *calls = g_tim.calls;
    if (main_ms) *main_ms = a;
    if (merge_ms) *merge_ms = b;
    g_tim.calls = 0;
    return ok();
}

pkv_status pkv_timing_collect_calls(int32_t* calls, float* main_ms, float* merge_ms, int32_t cap) {
    if (cap < 0 || (cap > 0 && (!main_ms || !merge_ms))) return fail(PKV_ERR_INVALID_ARG, "invalid timing buffers");
    for (int i = 0; i < g_tim.calls && i < cap; ++i) {
        pkv_status st = timing_of(i, main_ms[i], merge_ms[i]);
        if (st != PKV_OK) return st;
    }
    if (calls) *calls = g_tim.calls;
    g_tim.calls = 0;
    return ok();
}

}  // extern "C"
