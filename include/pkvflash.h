/*
 * pkvflash.h -- C ABI of the paged-KV FlashAttention library for MI355X (gfx950).
 *
 * Three operations, following the calls the "FlashAttention deep dive" page
 * (vLLM V1 FlashAttention backend) describes:
 *   pkv_cache_write        -- the KV-cache update by slot_mapping (core
 *                             implementation section, KV cache update);
 *   pkv_varlen_fwd         -- the varlen attention forward over a paged cache
 *                             addressed by a block table (core implementation
 *                             section, the varlen forward and its arguments);
 *                             semantics of the packed batch, the causal mask,
 *                             the online softmax, paging and split-KV follow
 *                             "How vLLM attention kernels handle multiple
 *                             requests in parallel", sections 1-12;
 *   pkv_merge_attn_states  -- the log-sum-exp merge of two attention states
 *                             (cascade attention section).
 *
 * Conventions for every call:
 *  - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *    caller owns every buffer. The library never allocates device memory,
 *    never synchronises the device and only enqueues work on `stream` (a
 *    hipStream_t; NULL is the default stream). Calls are therefore safe to
 *    capture into a HIP graph.
 *  - Tensors are dense and row-major in the layouts given below.
 *  - Arguments are validated on the host before anything is launched; on error
 *    nothing is enqueued, the return value names the class of error and
 *    pkv_last_error() gives a message (thread-local, valid until the next call
 *    on that thread).
 *  - Integer metadata (query_start_loc, seq_lens, block_table) lives on the
 *    device; its host-side summaries (num_tokens, max_seqlen_q, max_seqlen_k)
 *    size the launch so no device-to-host copy is needed. Values on the device
 *    that contradict them give undefined results.
 */
#ifndef PKVFLASH_H
#define PKVFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = 1,  /* a null pointer, a negative or inconsistent size */
    PKV_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement (dtype pair, head size) */
    PKV_ERR_WORKSPACE = 3,    /* the split-KV workspace is missing or too small */
    PKV_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} pkv_status;

/* Element types. PKV_FP8_E4M3FN is the OCP 8-bit float E4M3 ("fn": no
 * infinities, NaN = S.1111.111), the float8_e4m3fn type the deep-dive page's
 * FP8 section maps the "fp8" / "fp8_e4m3" cache dtypes to. */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3FN = 2 } pkv_dtype;

/* ------------------------------------------------------------------ cache write
 * For each new token t in [0, num_tokens):
 *   slot = slot_mapping[t]; if slot < 0 the token is padding and is skipped;
 *   block = slot / block_size, offset = slot % block_size;
 *   k_cache[block][offset][h][d] = enc(key[t][h][d]), likewise value -> v_cache.
 * Layouts: key, value [num_tokens, num_kv_heads, head_size] in src_dtype;
 *          k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_size]
 *          in cache_dtype (the K and V halves of the backend's
 *          (2, num_blocks, block_size, num_kv_heads, head_size) cache).
 *          slot_mapping [num_tokens] int64.
 * enc: same type -> bit copy; F32 -> BF16 round to nearest even;
 *      F32 or BF16 -> FP8_E4M3FN: y = x / scale as a correctly rounded binary32
 *      division by the per-tensor scale (*k_scale or *v_scale, device fp32
 *      scalars), then the nearest E4M3FN value, ties to even; |y| >= 448 and
 *      +-inf saturate to +-448; NaN gives 0x7F with the sign of y.
 * k_scale / v_scale are read only for an FP8 cache (may be NULL otherwise).
 * Two tokens with the same slot give an undefined result; every slot must be
 * < num_blocks * block_size (not checked on the device).
 * Errors: INVALID_ARG for null pointers or non-positive sizes, UNSUPPORTED for
 * other type pairs (BF16 -> F32, FP8 sources). num_tokens == 0 is a no-op.    */
pkv_status pkv_cache_write(const void* key, const void* value, pkv_dtype src_dtype,
                           void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                           const int64_t* slot_mapping, int64_t num_tokens,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int64_t num_blocks, const float* k_scale, const float* v_scale,
                           void* stream);

/* --------------------------------------------------------------- varlen forward
 * Attention over a packed batch of num_seqs requests. Request r owns query
 * tokens [query_start_loc[r], query_start_loc[r+1]) (q_len_r of them) and a KV
 * sequence of seq_lens[r] tokens that INCLUDES its q_len_r new tokens (their
 * K/V must already be in the cache: the cache write runs first). With
 * ctx_r = seq_lens[r] - q_len_r, query t of request r (request-local index)
 * sees keys 0 .. ctx_r + t when causal (bottom-right aligned mask, as in the
 * multi-token verification section), and every key 0 .. seq_lens[r]-1 when not.
 * Query head h reads kv head h / (num_heads / num_kv_heads) (GQA groups of
 * consecutive heads). Key j of request r is found through the block table:
 * block = block_table[r * block_table_stride + j / block_size], row
 * j % block_size of that block (paged address translation, section 11).
 *
 *   out[t][h] = sum_j softmax_j(softmax_scale * q[t][h] . k_j) v_j
 *   lse[h][t] = log(sum_j exp(softmax_scale * q[t][h] . k_j))   (natural log)
 * A row with no visible key gets out = 0 and lse = -inf.
 * Variants (the deep-dive page's table of supported variants names a sliding
 * window, a logits soft cap, attention sinks and ALiBi without formulas;
 * these are the plainest readings, each off by default):
 *   sliding_window > 0: the query at position i = ctx_r + t sees only the
 *          keys j >= i - (sliding_window - 1), at most sliding_window keys
 *          ending at its own position (on top of the causal bound); 0: no
 *          window (the zero of a cleared struct). KV tiles wholly before
 *          every query's window are not read.
 *   softcap > 0: each scaled score s becomes softcap * tanh(s / softcap)
 *          before the softmax; 0: no cap.
 *   sinks != NULL: sinks[h] (device fp32, [num_heads], natural-log units) is
 *          one more logit in head h's softmax normaliser that contributes no
 *          value row: out = sum_j e^{s_j} v_j / (e^{sink} + sum_j e^{s_j}) and
 *          lse = log(e^{sink} + sum_j e^{s_j}); a row with no visible key then
 *          gets out = 0, lse = sinks[h]. Split partials exclude the sink and
 *          the merge adds it once (a cascade passes sinks to one of its two
 *          forward calls only).
 *   alibi_slopes != NULL: alibi_slopes[h] (device fp32, [num_heads]) adds the
 *          linear position bias -alibi_slopes[h] * |i - j| to the score of
 *          query position i = ctx_r + t and key j, after the soft cap. The
 *          positions are those of the request's own sequence, so a cascade's
 *          prefix pass (which sees every query as one request) cannot carry it.
 *
 * Layouts: q, out [num_tokens, num_heads, head_size] in q_dtype (out has the
 *          type of q, except bf16 for an FP8_E4M3FN q); lse [num_heads,
 *          num_tokens] fp32, or NULL;
 *          k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_size]
 *          in kv_dtype; block_table int32 rows of block_table_stride entries
 *          (a row may be a strided view: pass the address of its first used
 *          entry and the stride of the full table); query_start_loc [num_seqs+1]
 *          and seq_lens [num_seqs] int32.
 * Flat mode: block_table == NULL means K and V are not paged: k_cache and
 *          v_cache are [num_tokens, num_kv_heads, head_size] packed like q and
 *          each request attends to its own new tokens only (seq_lens may be
 *          NULL; it is then taken as q_len).
 * Types:   q_dtype BF16 with kv_dtype BF16 or FP8_E4M3FN; F32 with F32;
 *          FP8_E4M3FN with FP8_E4M3FN (head_size 128 only). FP8 keys/values
 *          are multiplied by *k_scale / *v_scale, an FP8 q by *q_scale (device
 *          fp32), as the deep-dive page's backend passes q_descale, k_descale
 *          and v_descale to the forward (FP8 section). With an FP8 q the
 *          product Q K^T runs on the fp8 matrix cores (exact products, fp32
 *          sums) and P V on the bf16 ones (P rounded to bf16), whatever the
 *          shape of the batch.
 * Scales:  softmax_scale must be finite and > 0 (INVALID_ARG otherwise);
 *          the device scalars k_scale, v_scale and q_scale must be finite
 *          and > 0 (not checked: they live on the device).
 * Head size: a multiple of 8, at most 256 (the deep-dive page's backend rule).
 * Split-KV: num_splits 0 lets the library choose from the host sizes, 1 turns
 *          splitting off, > 1 asks for that many KV splits (at most 256). With
 *          more than one split the partial results (one per split) go to the
 *          workspace and a second kernel merges them by log-sum-exp
 *          (section 12); pkv_varlen_workspace_size gives the bytes needed.  */
typedef struct pkv_varlen_args {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    void* out;
    float* lse;
    const int32_t* query_start_loc;
    const int32_t* seq_lens;
    const int32_t* block_table;
    const float* k_scale;
    const float* v_scale;
    void* workspace;
    size_t workspace_bytes;
    int64_t block_table_stride;
    int64_t num_blocks;
    int64_t num_tokens;     /* query_start_loc[num_seqs], as a host integer */
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t head_size;
    int32_t block_size;
    int32_t max_seqlen_q;   /* >= every q_len_r */
    int32_t max_seqlen_k;   /* >= every seq_lens[r] */
    int32_t num_splits;
    int32_t causal;
    int32_t q_dtype;        /* pkv_dtype */
    int32_t kv_dtype;       /* pkv_dtype */
    float softmax_scale;
    /* attention variants (see above) */
    int32_t sliding_window; /* 0: no sliding window */
    float softcap;          /* 0: no logits soft cap */
    const float* sinks;     /* [num_heads] device fp32, or NULL */
    const float* q_scale;   /* FP8 q only: device fp32 */
    const float* alibi_slopes; /* [num_heads] device fp32, or NULL */
} pkv_varlen_args;

/* sizeof(pkv_varlen_args), so bindings can check their mirror of the struct. */
size_t pkv_varlen_args_size(void);

/* Validate `a` on the host only (no device access, no launch). */
pkv_status pkv_varlen_check(const pkv_varlen_args* a);

/* Number of KV partitions pkv_varlen_fwd will use for `a` (1 when the KV is
 * not split; 0 if the sizes in `a` are invalid), and the workspace bytes that
 * needs. Only the sizes, types and the block_table/NULL choice of `a` are
 * read: the data pointers may be NULL here. The workspace is caller-owned,
 * holds fp32 partial results and may be reused between calls on one stream.
 * Decode batches (max_seqlen_q * num_heads / num_kv_heads <= 16, at most 1024
 * requests) with num_splits == 0 use a balanced schedule: the 32-key KV tiles
 * of all requests and kv heads are dealt out in equal shares to a fixed set
 * of waves (the number returned), each writing a partial state per request
 * segment it covers, which the merge kernel combines; without a large enough
 * workspace such a batch runs unsplit. Other problems split each request's
 * KV into equal key ranges. */
int32_t pkv_varlen_num_splits(const pkv_varlen_args* a);
size_t pkv_varlen_workspace_size(const pkv_varlen_args* a);

pkv_status pkv_varlen_fwd(const pkv_varlen_args* a, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as pkv_varlen_fwd, same plan and kernels, with its split-KV partials
 * in a static device array of 64 MiB (67108864 bytes) inside the library
 * instead of a->workspace (ignored). Each GPU the library runs on holds its
 * own copy of the array until the process ends; its address is looked up on
 * the first call on each device (with that device current). The call
 * allocates nothing. Every call on a GPU shares that GPU's array and leaves
 * its partials there: calls that overlap on one GPU (several streams, several
 * threads) race and give undefined results. No kernel needs the array
 * cleared. Errors: as pkv_varlen_fwd, and WORKSPACE when the plan's partials
 * need more than the array holds (pkv_varlen_workspace_size(a) bytes; with
 * num_splits = 1 none are needed).                                          */
pkv_status pkv_varlen_fwd_noalloc(const pkv_varlen_args* a, void* stream);

/* ----------------------------------------------------------------------- merge
 * Merge two attention states of the same queries (cascade attention: a state
 * over the shared prefix and one over each request's own suffix):
 *   lse = log(exp(prefix_lse) + exp(suffix_lse))
 *   out = exp(prefix_lse - lse) * prefix_out + exp(suffix_lse - lse) * suffix_out
 * computed in fp32 with the larger lse subtracted first. A state whose lse is
 * -inf has weight 0; if both are -inf, out = 0 and lse = -inf.
 * Layouts: out, prefix_out, suffix_out [num_tokens, num_heads, head_size] in
 * dtype (BF16 or F32); prefix_lse, suffix_lse, out_lse [num_heads, num_tokens]
 * fp32; out_lse may be NULL. out may alias prefix_out or suffix_out.          */
pkv_status pkv_merge_attn_states(void* out, float* out_lse, const void* prefix_out, const float* prefix_lse,
                                 const void* suffix_out, const float* suffix_lse, int64_t num_tokens,
                                 int32_t num_heads, int32_t head_size, pkv_dtype dtype, void* stream);

/* ---------------------------------------------------------------- cascade
 * Cascade attention (deep-dive page, cascade attention section): when every
 * request of a batch begins with the same common_prefix_len KV tokens on the
 * same pages, the batch runs as
 *   1. a prefix pass: every query token of the batch against the shared
 *      prefix (the first common_prefix_len / block_size pages of the first
 *      block-table row), with no causal mask, as one request;
 *   2. a suffix pass: each request against its own keys past the prefix (its
 *      block-table row from page common_prefix_len / block_size on, KV length
 *      seq_lens[r] - common_prefix_len), with the batch's mask;
 *   3. pkv_merge_attn_states of the two states into a->out (and a->lse).
 * The result equals pkv_varlen_fwd over the whole batch, with the shared
 * pages read once instead of once per request.
 * When the whole batch fits one item of the balanced decode (bf16 q,
 * num_tokens x the group at most 16 query rows, or 32 with head size up to
 * 128), the three steps run as one decode launch and one merge launch: the
 * prefix pass joins the decode's tile list as a further request, and the
 * merge folds its partial states into each row with the suffix's.
 * `a` describes the whole batch exactly as for pkv_varlen_fwd (block_table
 * required); both passes and the merge run inside the library on `stream`.
 * Preconditions (device data, not checked): every request's first
 * common_prefix_len block-table entries are the same pages, and, with the
 * causal mask, every request has at least common_prefix_len keys before its
 * first query token (seq_lens[r] - q_len_r >= common_prefix_len), so each of
 * its queries sees the whole prefix. Results are undefined otherwise (the
 * kernels stay inside the pages the table names).
 * Sinks (a->sinks) join the suffix pass only, so the merged normaliser counts
 * them once. Not supported (UNSUPPORTED): ALiBi (its bias needs each query's
 * own position, which the one-request prefix pass does not keep) and a
 * sliding window (the deep-dive page's decision rules cascades out for it).
 * Workspace: a->workspace must hold pkv_cascade_workspace_size(a, P) bytes
 * (caller-owned): both passes' outputs and lse, and their split partials.
 * common_prefix_len must be a positive multiple of block_size and at most
 * max_seqlen_k (INVALID_ARG otherwise); WORKSPACE if the workspace is short.
 * pkv_cascade_workspace_size returns 0 for arguments it rejects.            */
size_t pkv_cascade_workspace_size(const pkv_varlen_args* a, int32_t common_prefix_len);
pkv_status pkv_cascade_fwd(const pkv_varlen_args* a, int32_t common_prefix_len, void* stream);

/* Whether to run a batch whose requests share their first common_prefix_len
 * KV tokens (the same pages) as a cascade (pkv_cascade_fwd) rather than
 * plainly (pkv_varlen_fwd). The deep-dive page's decision (cascade attention
 * section) first rules it out for a prefix under 256 tokens and for sliding
 * windows; its remaining test, a performance model, is not printed, and its
 * request-count rule (fewer than 8 requests: no) is that model's stand-in for
 * its own kernels. Here a model of this library's decode kernels takes both
 * places, fitted to MI355X measurements of 24 shared-prefix decode batches
 * (1 to 64 requests, 2K to 256K keys): the plain form reads the unique keys
 * (the prefix once, every suffix) at 5.6 TB/s plus 17 us, and of its
 * re-reads of the shared pages (once per further request) a share reaches
 * HBM that grows with the prefix's part of the mean KV length f: 0 up to
 * f = 0.2, then 2.4 (f - 0.2), at most 0.6 (the last-level cache serves the
 * rest, as far as the requests' reads of a page fall close in time); the
 * cascade reads the unique keys only, at 5.8 TB/s plus 32 us as one launch
 * (see pkv_cascade_fwd: num_tokens and num_heads decide whether it applies,
 * for a bf16 q) and at 5.5 TB/s plus 40 us as three. Bytes per key:
 * num_kv_heads * head_size * 2 * element bytes.
 * host_seq_lens: num_seqs KV lengths in host memory; num_tokens: query tokens
 * of the batch. Writes 1 (cascade) or 0 to *use_cascade and, when not NULL,
 * the two predicted times in us. INVALID_ARG for negative sizes or lengths,
 * num_heads not a positive multiple of num_kv_heads, or NULL use_cascade.    */
pkv_status pkv_cascade_choose(int32_t common_prefix_len, int32_t num_seqs, const int32_t* host_seq_lens,
                              int64_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                              pkv_dtype kv_dtype, int32_t sliding_window, int32_t* use_cascade, double* t_plain_us,
                              double* t_cascade_us);

/* ------------------------------------------------------------------ utilities */

/* Message for the last error on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pkv_version(void);

/* Kernel timing. When enabled, every pkv_varlen_fwd call records HIP events
 * around its main attention kernel and around its split-merge kernel, on the
 * call's stream (at most 4096 calls are kept; later ones are not recorded).
 * pkv_timing_collect waits for the recorded events, returns the number of
 * calls and the summed milliseconds of each kernel, and clears the record.
 * Enabling creates the events (it is the only call that allocates); disabling
 * releases them. Not thread-safe. pkv_timing_collect_calls does the same but
 * writes each call's milliseconds (main kernel, merge kernel or 0) to the
 * host arrays main_ms / merge_ms, at most cap entries, in call order.       */
pkv_status pkv_timing_enable(int32_t on);
pkv_status pkv_timing_collect(int32_t* calls, double* main_ms, double* merge_ms);
pkv_status pkv_timing_collect_calls(int32_t* calls, float* main_ms, float* merge_ms, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PKVFLASH_H */
