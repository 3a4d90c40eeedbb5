/*
 * mimo_attn.h -- C ABI of the MI355X (gfx950) MiMo-V2-Flash hybrid attention library.
 *
 * The operation (Hugging Face Transformers model doc "MiMo-V2-Flash"):
 *   - Key features: sliding-window attention (SWA) and global attention (GA)
 *     layers alternate 5:1; the window is 128 tokens; a learnable attention
 *     sink bias keeps long-context quality.
 *   - MiMoV2FlashConfig: num_attention_heads (64), num_key_value_heads (4,
 *     grouped-query attention), head_dim (192, queries and keys), v_head_dim
 *     (128), sliding_window (129), attention_value_scale (0.707).
 *   - MiMoV2FlashModel.forward / past_key_values: a cache holds the keys and
 *     values of earlier tokens, and with a cache only the unprocessed tokens are
 *     passed.  The decoder is causal (MiMoV2FlashForCausalLM).
 *
 * For a query token at position p of its sequence and query head h, with
 * G = num_q_heads / num_kv_heads and g = h / G:
 *   keys       j in [lo, p],  lo = 0 (GA)  or  max(0, p - (sliding_window - 1)) (SWA)
 *   s_j        = softmax_scale * dot(q[p,h,:], k[j,g,:])
 *   M          = max(max_j s_j, sink[h])            (sink left out when absent)
 *   Z          = sum_j exp(s_j - M) + exp(sink[h] - M)
 *   lse[p,h]   = M + ln Z                            (natural log, sink included)
 *   out[p,h,e] = value_scale * sum_j exp(s_j - lse) * v[j,g,e]
 * The sink joins the softmax denominator only; it has no value row.  A NULL
 * sink pointer, or a sink value of -inf, means "no sink".
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device unless
 *     marked (host).  bf16 tensors are passed as uint16_t bit patterns.
 *   - Layouts are dense, row-major, token-major:
 *       q   [T][Hq][192]     k [T][Hkv][192]     v [T][Hkv][128]
 *       out [T][Hq][128]     lse [T][Hq] (fp32)  sink [Hq] (fp32)
 *     Every tensor must be 16-byte aligned.
 *   - The caller allocates and owns every buffer (caches, workspace included).
 *     The library allocates nothing, never synchronises the device (check
 *     mode aside) and never writes ctx_lens.  Its state between calls: a
 *     per-thread copy of the last failure's message (mimo_last_error), the
 *     check-mode switch and per-device word, and the no-allocation decode's
 *     scratch array; no computed result depends on them.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *   - Misuse detectable on the host returns a status BEFORE anything is
 *     enqueued.  A failed launch returns MIMO_ERR_HIP.  mimo_last_error()
 *     gives a message for the calling thread's most recent failure.
 *   - Supported shapes: head_dim_qk == 192, head_dim_v == 128 and
 *     num_q_heads == 16 * num_kv_heads <= 65535; anything else is
 *     MIMO_ERR_UNSUPPORTED.
 *   - Inputs must be finite.  Device-resident preconditions (monotone
 *     cu_seqlens, ctx_lens within the stated bounds, ...) are not checked on
 *     the device except where an entry point says so, or in check mode.
 *   - Check mode (environment MIMO_ATTN_CHECK=1 when the library is first
 *     called, or mimo_attn_set_check): every call that reads device-resident
 *     sizes, offsets, block tables, sinks or FP8 scales first enqueues a
 *     check of them (the MIMO_CHECK_* rules below).  Outside graph capture
 *     the call then waits for its stream and, on a violation, returns
 *     MIMO_ERR_PRECONDITION without enqueuing its own kernels.  Under capture
 *     the check joins the graph and only records its findings: the call's
 *     kernels are captured too.  Findings also accumulate in a sticky word
 *     per device, read with mimo_attn_check_flags.  Meant for debugging: it
 *     synchronises, and concurrent checked calls on one device share the
 *     word that reports the latest check.
 *   - Calls are reentrant; calls on different streams may run concurrently
 *     when their output buffers do not overlap.
 */
#ifndef MIMO_ATTN_H
#define MIMO_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIMO_ATTN_ABI_VERSION 14

/* Layer type: which key set a query sees (model doc, Key features; config
 * layer_types). */
typedef enum {
    MIMO_LAYER_SWA = 0, /* keys p-(sliding_window-1) .. p */
    MIMO_LAYER_GA = 1   /* keys 0 .. p (global causal)    */
} mimo_layer_type;

typedef enum {
    MIMO_OK = 0,
    MIMO_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, bad layer type ... */
    MIMO_ERR_UNSUPPORTED = 2, /* shape outside the specialised kernels        */
    MIMO_ERR_WORKSPACE = 3,   /* decode workspace missing or too small         */
    MIMO_ERR_HIP = 4,         /* a HIP launch or query failed                  */
    MIMO_ERR_PRECONDITION = 5 /* check mode: a device-resident argument breaks
                                 its contract (MIMO_CHECK_* bits)              */
} mimo_status;

/* Check-mode findings, one bit per rule. */
#define MIMO_CHECK_CU_START    0x001u /* cu_seqlens[0] != 0                            */
#define MIMO_CHECK_CU_ORDER    0x002u /* cu_seqlens decreases somewhere                */
#define MIMO_CHECK_CU_LENGTH   0x004u /* a sequence longer than max_seqlen / max_newlen */
#define MIMO_CHECK_CU_TOTAL    0x008u /* cu_seqlens[num_seqs] != total_tokens / total_new */
#define MIMO_CHECK_CTX_RANGE   0x010u /* ctx_lens[b] < 0, above max_ctx, or ctx + new
                                         positions past INT32_MAX                     */
#define MIMO_CHECK_KV_BASE     0x020u /* kv_base[b] < 0                                */
#define MIMO_CHECK_CAPACITY    0x040u /* ctx + new above kv_capacity[b], or positions
                                         past max_blocks * page_size                  */
#define MIMO_CHECK_BLOCK_TABLE 0x080u /* a block entry the call reads or writes is
                                         outside [0, num_pages)                       */
#define MIMO_CHECK_SINK        0x100u /* a sink value is NaN or +inf                   */
#define MIMO_CHECK_FP8_SCALE   0x200u /* an FP8 scale is not positive and finite       */

/* Attention shape, mirroring MiMoV2FlashConfig (model doc, MiMoV2FlashConfig):
 * num_attention_heads, num_key_value_heads, head_dim, v_head_dim,
 * sliding_window and attention_value_scale; softmax_scale is 1/sqrt(head_dim)
 * for the model.  Passed by host pointer. */
typedef struct {
    int32_t num_q_heads;    /* Hq  = 64                                       */
    int32_t num_kv_heads;   /* Hkv = 4; Hq / Hkv must be 16                   */
    int32_t head_dim_qk;    /* 192                                            */
    int32_t head_dim_v;     /* 128                                            */
    int32_t sliding_window; /* W = 129: SWA keys p-(W-1)..p; ignored for GA   */
    float softmax_scale;    /* multiplies q.k; 1/sqrt(192) for the model      */
    float value_scale;      /* multiplies the output; 1.0, or 0.707 for the   */
                            /* model's attention_value_scale                  */
} mimo_attn_dims;

/*
 * Prefill: attention of every token of num_seqs packed variable-length
 * sequences over keys of its own sequence (model doc, MiMoV2FlashModel.forward:
 * a batch of sequences without a cache; padding replaced by packing).
 *
 *   q, k, v      packed tokens, layouts above; sequence b owns tokens
 *                cu_seqlens[b] .. cu_seqlens[b+1]-1 and its positions start at 0.
 *   cu_seqlens   [num_seqs+1] int32 (device), cu_seqlens[0] == 0, non-decreasing.
 *   num_seqs     >= 1 (host).
 *   max_seqlen   (host) >= every sequence length; sizes the grid.  Tokens of a
 *                longer sequence beyond max_seqlen are left unwritten.
 *   sink         [Hq] fp32 (device) or NULL.
 *   out          [T][Hq][128] bf16, rounded to nearest even.
 *   lse          [T][Hq] fp32, or NULL to skip it.
 * A call with max_seqlen == 0 enqueues nothing and returns MIMO_OK.
 */
int mimo_attn_prefill(const mimo_attn_dims* dims, int layer_type,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                      const float* sink, uint16_t* out, float* lse, hipStream_t stream);

/*
 * Chunked prefill: attention of new tokens that continue cached sequences
 * (model doc, MiMoV2FlashModel.forward, past_key_values: with a cache only the
 * unprocessed tokens are passed).  New token i of sequence b sits at position
 * p = ctx_lens[b] + i and sees keys lo..p (lo as above): positions below
 * ctx_lens[b] are read from the cache, the others from this call's k, v.
 *
 *   q, k, v      packed new tokens [Tn][Hq][192], [Tn][Hkv][192], [Tn][Hkv][128].
 *   cu_newlens   [num_seqs+1] int32 (device), cu_newlens[0] == 0, non-decreasing.
 *   num_seqs     >= 1 (host).
 *   max_newlen   (host) >= every chunk length; tokens of a longer chunk beyond
 *                max_newlen are left unwritten.
 *   k_cache, v_cache, kv_base  as for mimo_attn_decode (SWA ring of W-1 slots
 *                per sequence, W >= 2; GA pool with base rows kv_base[b]).
 *   ctx_lens     [num_seqs] int32 (device): positions already cached.  For GA,
 *                pool rows kv_base[b] .. kv_base[b] + ctx_lens[b] - 1 are read;
 *                for SWA the ring must hold positions max(0, ctx_lens[b]-(W-1))
 *                .. ctx_lens[b]-1 (what mimo_kv_append leaves behind).
 *   sink, out, lse  as for prefill, with T = Tn; lse may be NULL.
 * The cache is only read.  Order: attend, then append the chunk with
 * mimo_kv_append (same cu_newlens and ctx_lens) -- for SWA the append may
 * overwrite ring slots this call still reads.
 * A call with max_newlen == 0 enqueues nothing and returns MIMO_OK.
 */
int mimo_attn_prefill_chunk(const mimo_attn_dims* dims, int layer_type,
                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                            const uint16_t* k_cache, const uint16_t* v_cache,
                            const int64_t* kv_base, const int32_t* ctx_lens,
                            const float* sink, uint16_t* out, float* lse, hipStream_t stream);

/*
 * Bytes of device workspace mimo_attn_decode needs for these arguments.  SWA
 * needs none (returns 0).  GA splits the keys of all sequences into chunks of
 * 32-key units (see mimo_attn_decode) and needs a header of batch + 2 int64,
 * padded to 256 bytes, plus (chunks + batch) * Hq * 130 * 4 bytes of partial
 * results, where chunks is at most 256 (so the size does not grow with
 * max_ctx beyond that).  split_tokens <= 0 selects the default.  Returns 0 for
 * arguments mimo_attn_decode would reject.
 */
size_t mimo_attn_decode_workspace_size(const mimo_attn_dims* dims, int layer_type,
                                       int32_t batch, int32_t max_ctx, int32_t split_tokens);

/*
 * Decode: attention of ONE new token per sequence, at position p = ctx_lens[b],
 * over cached keys and itself (model doc, past_key_values: only the
 * unprocessed token is passed; earlier keys come from the cache).
 *
 *   q            [batch][Hq][192] bf16, the new tokens' queries.
 *   k_new, v_new [batch][Hkv][192], [batch][Hkv][128]: the new tokens' key and
 *                value (position p is read from here, not from the cache).
 *   k_cache, v_cache
 *                SWA: ring [batch][W-1][Hkv][192], [batch][W-1][Hkv][128];
 *                     position j of sequence b lives in slot j mod (W-1).
 *                GA:  pool [N][Hkv][192], [N][Hkv][128]; position j of
 *                     sequence b lives in row kv_base[b] + j.
 *   kv_base      GA: [batch] int64 (device); SWA: ignored (may be NULL).
 *   ctx_lens     [batch] int32 (device): tokens already cached; 0 <= p <= max_ctx.
 *   batch        >= 1 (host).
 *   max_ctx      (host) >= every ctx_lens[b]; bounds the GA split grid.  A GA
 *                sequence with ctx_lens[b] > max_ctx gets NaN outputs.
 *   split_tokens GA: the least number of keys per split chunk (host), rounded
 *                up to a multiple of 32; <= 0 selects 256.  GA splits the key
 *                space of the whole batch -- per sequence ceil(p/32) tiles of
 *                32 cached keys plus one unit for the new token -- into equal
 *                chunks, one per split workgroup: 256 chunks (one per compute
 *                unit of the part) when they hold at least split_tokens keys
 *                each, else chunks of split_tokens keys; a chunk may cover
 *                pieces of several sequences.  The plan is derived on the
 *                device from ctx_lens, so no workgroup is launched for keys
 *                that do not exist.  Results do not depend on it beyond fp32
 *                rounding.
 *   sink, out, lse  as for prefill, with T = batch; lse may be NULL.
 *   workspace    device buffer of >= mimo_attn_decode_workspace_size(...) bytes
 *                (GA only; NULL allowed for SWA).  Its contents need no
 *                initialisation and are scratch after the call.
 * Order for a decode step is attend, then append: this call reads cache
 * positions < p only, so the caller appends position p (mimo_kv_append) after
 * it.  For SWA this order is required, because slot p mod (W-1) still holds
 * position p-(W-1), which query p needs.
 */
int mimo_attn_decode(const mimo_attn_dims* dims, int layer_type,
                     const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                     const uint16_t* k_cache, const uint16_t* v_cache,
                     const int64_t* kv_base, const int32_t* ctx_lens,
                     int32_t batch, int32_t max_ctx, int32_t split_tokens,
                     const float* sink, uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mimo_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of mimo_attn_decode (split_tokens included); the GA plan header and partial
 * results live in a 32 MiB device array inside the library, one per GPU the
 * library runs on, held until the process ends (its address is looked up
 * once per device, on the first call there).  The call itself allocates and
 * frees nothing.  Limit: the plan needs a 256-byte-padded header of batch + 2
 * int64 plus (chunks + batch) slots of Hq * 520 bytes within the 32 MiB; the
 * chunk count is capped to fit (results then differ from mimo_attn_decode
 * only by fp32 rounding), and a batch too large for even one chunk is
 * MIMO_ERR_UNSUPPORTED (with 64 query heads, up to about 1,000 sequences fit).
 * SWA needs no scratch.  Every call on a GPU shares that GPU's array: calls
 * that overlap in time on one GPU (concurrent streams, threads) race and give
 * wrong results; serialise them.
 */
int mimo_attn_decode_noalloc(const mimo_attn_dims* dims, int layer_type,
                             const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                             const uint16_t* k_cache, const uint16_t* v_cache,
                             const int64_t* kv_base, const int32_t* ctx_lens,
                             int32_t batch, int32_t max_ctx, int32_t split_tokens,
                             const float* sink, uint16_t* out, float* lse, hipStream_t stream);

/*
 * KV append: writes new tokens' keys and values into the caches (model doc,
 * past_key_values / use_cache).  New token i of sequence b has position
 * ctx_lens[b] + i.
 *
 *   k, v         packed new tokens [Tn][Hkv][192], [Tn][Hkv][128] bf16.
 *   cu_newlens   [batch+1] int32 (device): sequence b owns new tokens
 *                cu_newlens[b] .. cu_newlens[b+1]-1 (prefill: cu_seqlens with
 *                ctx_lens all 0; decode step: 0,1,..,batch).
 *   ctx_lens     [batch] int32 (device): positions already cached.
 *   batch        >= 1 (host).
 *   total_new    (host) == cu_newlens[batch]; sizes the grid.
 *   k_cache, v_cache  as for decode.
 *   kv_base, kv_capacity  GA: [batch] int64 (device) -- sequence b may use pool
 *                rows kv_base[b] .. kv_base[b] + kv_capacity[b] - 1.  A
 *                sequence whose ctx_lens[b] + new tokens exceeds its capacity is
 *                skipped entirely (nothing written for it).  SWA: ignored.
 * SWA keeps, per sequence, only the last W-1 positions: a token is written to
 * slot position mod (W-1) when position >= ctx_lens[b] + n_b - (W-1).
 * Repeating a call with the same arguments writes the same bytes.
 */
int mimo_kv_append(const mimo_attn_dims* dims, int layer_type,
                   const uint16_t* k, const uint16_t* v,
                   const int32_t* cu_newlens, const int32_t* ctx_lens,
                   int32_t batch, int32_t total_new,
                   uint16_t* k_cache, uint16_t* v_cache,
                   const int64_t* kv_base, const int64_t* kv_capacity, hipStream_t stream);

/*
 * One decode step with its append in the same launch: the result, the
 * outputs and the caches afterwards are those of mimo_attn_decode followed by
 * mimo_kv_append of the one new token per sequence (cu_newlens = 0, 1, ...,
 * batch; position ctx_lens[b]).  For the many small decode calls of a layer
 * stack this saves the append's separate launch.
 *
 * Arguments as for mimo_attn_decode, with k_cache / v_cache writable, plus
 *   kv_capacity  GA: [batch] int64 (device), rows reserved for sequence b; the
 *                new row kv_base[b] + p is written only when p < kv_capacity[b]
 *                (as mimo_kv_append refuses a sequence that would overflow).
 *                SWA: ignored (may be NULL).
 * The SWA workgroup of (b, KV head) writes ring slot p mod (W-1) after all of
 * its own reads of the ring (that slot still holds position p-(W-1), which
 * query p attends to).  The GA row p is not read by the attention of this
 * call.  bf16 caches only (the paged and FP8 pools keep separate calls).
 * ctx_lens is not advanced.  Errors as for mimo_attn_decode; GA without
 * kv_base or kv_capacity is MIMO_ERR_INVALID_ARG.
 */
int mimo_attn_decode_append(const mimo_attn_dims* dims, int layer_type,
                            const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                            uint16_t* k_cache, uint16_t* v_cache,
                            const int64_t* kv_base, const int64_t* kv_capacity, const int32_t* ctx_lens,
                            int32_t batch, int32_t max_ctx, int32_t split_tokens,
                            const float* sink, uint16_t* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Paged GA pool.  The cache of past_key_values (model doc,
 * MiMoV2FlashModel.forward) for a GA layer may live in fixed-size pages of one
 * shared pool instead of one contiguous range per sequence; paging is a
 * serving layout of the same cache and changes nothing that is computed.
 *
 *   k_cache, v_cache  [num_pages * page_size][Hkv][192], [...][Hkv][128] bf16:
 *                page n is rows n*page_size .. n*page_size + page_size - 1.
 *   block_table  [batch][max_blocks] int32 (device): entry [b][i] is the page
 *                holding positions i*page_size .. i*page_size + page_size - 1
 *                of sequence b, so position j lives in row
 *                block_table[b][j / page_size] * page_size + j % page_size.
 *   page_size    tokens per page (host): a power of two in [16, 65536].
 *   max_blocks   columns of block_table (host), >= 1.
 *   num_pages    pages in the pool (host), >= 1.
 * Entries for blocks a call reads must lie in [0, num_pages).  An entry
 * outside that range is never dereferenced: decode reads its keys as zero
 * vectors, chunked prefill reads them from page 0, append skips the tokens on
 * it -- the results for that sequence are then meaningless, but no memory
 * outside the pool is touched.  Passed by host pointer.
 */
typedef struct {
    const int32_t* block_table;
    int32_t max_blocks;
    int32_t page_size;
    int64_t num_pages;
} mimo_kv_pages;

/*
 * mimo_kv_append for a GA layer whose cache is a paged pool: position pos of
 * sequence b is written to row block_table[b][pos / page_size] * page_size +
 * pos % page_size.  A sequence whose ctx_lens[b] + new tokens exceeds
 * max_blocks * page_size is skipped entirely; a token whose block entry is
 * outside [0, num_pages) is not written.  Other arguments as mimo_kv_append.
 */
int mimo_kv_append_paged(const mimo_attn_dims* dims,
                         const uint16_t* k, const uint16_t* v,
                         const int32_t* cu_newlens, const int32_t* ctx_lens,
                         int32_t batch, int32_t total_new,
                         uint16_t* k_cache, uint16_t* v_cache,
                         const mimo_kv_pages* pages, hipStream_t stream);

/*
 * GA decode (as mimo_attn_decode with layer_type GA) over a paged pool.  The
 * workspace is mimo_attn_decode_workspace_size(dims, MIMO_LAYER_GA, batch,
 * max_ctx, split_tokens) bytes.  Results are bit-identical to
 * mimo_attn_decode over a contiguous pool holding the same rows.
 */
int mimo_attn_decode_paged(const mimo_attn_dims* dims,
                           const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                           const uint16_t* k_cache, const uint16_t* v_cache,
                           const mimo_kv_pages* pages, const int32_t* ctx_lens,
                           int32_t batch, int32_t max_ctx, int32_t split_tokens,
                           const float* sink, uint16_t* out, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * GA chunked prefill (as mimo_attn_prefill_chunk with layer_type GA) whose
 * cached positions live in a paged pool.  Results are bit-identical to
 * mimo_attn_prefill_chunk over a contiguous pool holding the same rows.
 */
int mimo_attn_prefill_chunk_paged(const mimo_attn_dims* dims,
                                  const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const mimo_kv_pages* pages, const int32_t* ctx_lens,
                                  const float* sink, uint16_t* out, float* lse, hipStream_t stream);

/*
 * FP8 GA pool.  A storage format of the same GA cache (the model doc defines
 * none): OCP 8-bit floating point E4M3 codes ("OCP 8-bit Floating Point
 * Specification (OFP8)": bias 7, largest finite 448, S.1111.111 = NaN, no
 * infinities), half the bytes of the bf16 pool.  Each KV head g has one fp32
 * scale for keys (k_scale[g]) and one for values (v_scale[g]): element x of
 * head g is stored as E4M3(clamp(x / scale[g], -448, 448)) -- the division in
 * fp32 (IEEE), the rounding to nearest-even -- and read back as
 * value(code) * scale[g].
 *
 *   k_cache, v_cache  pool [N][Hkv][192] and [N][Hkv][128] of uint8 codes;
 *                position j of sequence b lives in row kv_base[b] + j.
 *   k_scale, v_scale  [Hkv] fp32 (device), positive and finite.
 */

/*
 * mimo_kv_append for a GA layer whose cache is an FP8 pool: new tokens are
 * quantised as above into rows kv_base[b] + position; capacity as for
 * mimo_kv_append (a sequence past kv_capacity[b] is skipped entirely).
 */
int mimo_kv_append_fp8(const mimo_attn_dims* dims,
                       const uint16_t* k, const uint16_t* v,
                       const int32_t* cu_newlens, const int32_t* ctx_lens,
                       int32_t batch, int32_t total_new,
                       uint8_t* k_cache, uint8_t* v_cache,
                       const int64_t* kv_base, const int64_t* kv_capacity,
                       const float* k_scale, const float* v_scale, hipStream_t stream);

/*
 * GA decode (as mimo_attn_decode with layer_type GA) over an FP8 pool: cached
 * positions j < p are read as value(code) * scale; the new token at p is read
 * from k_new / v_new (bf16) as given.  Workspace: mimo_attn_decode_workspace_size
 * (dims, MIMO_LAYER_GA, batch, max_ctx, split_tokens) bytes.
 */
int mimo_attn_decode_fp8(const mimo_attn_dims* dims,
                         const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* kv_base,
                         const float* k_scale, const float* v_scale, const int32_t* ctx_lens,
                         int32_t batch, int32_t max_ctx, int32_t split_tokens,
                         const float* sink, uint16_t* out, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The FP8 GA pool in the other cache layouts (ABI version 11); codes and
 * scales exactly as above, results bit-identical to the bf16 entry points'
 * treatment of the same layout wherever the dequantised values are exact.
 *
 * mimo_kv_append_fp8_paged: as mimo_kv_append_paged (rows through the block
 * table; a sequence past max_blocks * page_size skipped whole, a token on a
 * block outside [0, num_pages) not written), storing E4M3 codes.
 *
 * mimo_attn_decode_fp8_paged: as mimo_attn_decode_fp8 with the code rows of
 * position j of sequence b in row block_table[b][j / P] * P + j mod P
 * (mimo_kv_pages, passed by host pointer); workspace as for
 * mimo_attn_decode_fp8.
 *
 * mimo_attn_prefill_chunk_fp8 / _fp8_paged: GA chunked prefill
 * (mimo_attn_prefill_chunk, mimo_attn_prefill_chunk_paged) whose cached
 * positions j < ctx_lens[b] are read from an FP8 pool as value(code) *
 * scale[g]; the chunk's own keys and values (k, v) are bf16 as given.
 */
int mimo_kv_append_fp8_paged(const mimo_attn_dims* dims,
                             const uint16_t* k, const uint16_t* v,
                             const int32_t* cu_newlens, const int32_t* ctx_lens,
                             int32_t batch, int32_t total_new,
                             uint8_t* k_cache, uint8_t* v_cache, const mimo_kv_pages* pages,
                             const float* k_scale, const float* v_scale, hipStream_t stream);

int mimo_attn_decode_fp8_paged(const mimo_attn_dims* dims,
                               const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                               const uint8_t* k_cache, const uint8_t* v_cache, const mimo_kv_pages* pages,
                               const float* k_scale, const float* v_scale, const int32_t* ctx_lens,
                               int32_t batch, int32_t max_ctx, int32_t split_tokens,
                               const float* sink, uint16_t* out, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

int mimo_attn_prefill_chunk_fp8(const mimo_attn_dims* dims,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                                const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* kv_base,
                                const float* k_scale, const float* v_scale, const int32_t* ctx_lens,
                                const float* sink, uint16_t* out, float* lse, hipStream_t stream);

int mimo_attn_prefill_chunk_fp8_paged(const mimo_attn_dims* dims,
                                      const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen,
                                      const uint8_t* k_cache, const uint8_t* v_cache, const mimo_kv_pages* pages,
                                      const float* k_scale, const float* v_scale, const int32_t* ctx_lens,
                                      const float* sink, uint16_t* out, float* lse, hipStream_t stream);

/*
 * Backward of mimo_attn_prefill: the gradients of sum(dout * out) for an
 * upstream gradient dout, including the learnable sink's (model doc, Key
 * features: the sink bias is learnable).  With P_j = exp(s_j - lse) for the
 * query row's keys j (lse natural log, sink included) and o the row's output:
 *   D     = dout . o                     dP_j = value_scale * dout . v_j
 *   dS_j  = P_j * (dP_j - D)
 *   dq    = softmax_scale * sum_j dS_j k_j
 *   dk_j  = softmax_scale * sum over rows seeing j (16 heads of the group) of dS_j q
 *   dv_j  = value_scale * sum over those rows of P_j dout
 *   dsink[h] = -sum over tokens of exp(sink[h] - lse) * D
 *
 *   q, k, v, cu_seqlens, num_seqs, max_seqlen, sink  as for the forward call.
 *   out, lse     the forward's out [T][Hq][128] bf16 and lse [T][Hq] fp32 (required).
 *   dout         [T][Hq][128] bf16.
 *   total_tokens (host) == cu_seqlens[num_seqs]; sizes the workspace.
 *   dq, dk, dv   [T][Hq][192], [T][Hkv][192], [T][Hkv][128] bf16, rounded to
 *                nearest even.  Rows of tokens past max_seqlen are left
 *                unwritten, and such tokens contribute nothing.
 *   dsink        [Hq] fp32, or NULL to skip; all zero when sink is NULL.
 *   workspace    >= mimo_attn_prefill_backward_workspace_size(dims,
 *                total_tokens) bytes of device memory, no initialisation.
 * A call with max_seqlen == 0 or total_tokens == 0 computes no rows (dq, dk
 * and dv are left unwritten) and needs no workspace; it writes dsink, when
 * given, as zeros (a sum over no tokens).
 */
size_t mimo_attn_prefill_backward_workspace_size(const mimo_attn_dims* dims, int32_t total_tokens);

int mimo_attn_prefill_backward(const mimo_attn_dims* dims, int layer_type,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* out, const float* lse, const uint16_t* dout,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                               int32_t total_tokens, const float* sink,
                               uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dsink,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Rotary position embedding of queries and keys, in place, before attention
 * and append (model doc, MiMoV2FlashConfig: rope_parameters with rope_theta,
 * the Transformers rotary convention; the pages give neither theta nor how
 * many dims rotate, so both come from the caller).  For a head vector x of the
 * token at position p, the first rd = rotary_dim dims rotate in pairs
 * (i, i + rd/2), i < rd/2, by the angle p * theta^(-2i/rd):
 *   x[i] <- x[i] cos - x[i + rd/2] sin,  x[i + rd/2] <- x[i + rd/2] cos + x[i] sin
 * and the other dims are left as they are.
 *
 *   q, k         [T][Hq][192] and [T][Hkv][192] bf16, rotated in place (either
 *                may be NULL, not both).  Results round to nearest even.
 *   positions    [T] int32 (device): position of each token (prefill: 0..L-1
 *                per sequence; a chunk: ctx_lens[b] + i; decode: ctx_lens[b]).
 *   rope_theta   > 1 (host); rotary_dim in [0, 192], a multiple of 16 (host;
 *                0 does nothing).  Angles are formed in fp64.
 */
int mimo_rope_apply(const mimo_attn_dims* dims, uint16_t* q, uint16_t* k, const int32_t* positions,
                    int32_t total_tokens, float rope_theta, int32_t rotary_dim, hipStream_t stream);

/*
 * Prefill with the rotary embedding fused in (model doc, MiMoV2FlashConfig:
 * rope_parameters / rope_theta; MiMoV2FlashModel.forward: position_ids): the
 * result is that of mimo_rope_apply on copies of q and k followed by
 * mimo_attn_prefill, bit for bit, without the separate pass over q.  Q is
 * rotated as the attention kernels load it; K is rotated once, by a pass over
 * K alone that also forms each token's cos/sin table, into k_rot, which the
 * attention reads and the caller then appends (mimo_kv_append), so that the
 * caches hold post-RoPE keys.
 *
 *   q, k, v        as for mimo_attn_prefill, before the rotation; q, k and v
 *                  are only read (k_rot == k is allowed and rotates k in place).
 *   positions      [total_tokens] int32 (device): the position id of each
 *                  packed token (0 .. L-1 within a sequence for a plain
 *                  prefill); positions only steer the rotation, the masks use
 *                  token order as for mimo_attn_prefill.
 *   total_tokens   (host) == cu_seqlens[num_seqs].
 *   rope_theta     > 1 (host); rotary_dim a multiple of 32 in [32, 192] (host):
 *                  the pairs (i, i + rotary_dim/2) rotate by the angle
 *                  p * theta^(-2i/rotary_dim), formed in fp64, as for
 *                  mimo_rope_apply; other rotary_dim values are
 *                  MIMO_ERR_UNSUPPORTED (use mimo_rope_apply).
 *   k_rot          [total_tokens][Hkv][192] bf16 (device): K after the rotation.
 *   workspace      >= mimo_attn_prefill_rope_workspace_size(dims, total_tokens,
 *                  rotary_dim) bytes of device memory (the tokens' fp32 cos/sin
 *                  table), no initialisation, scratch after the call.
 * A call with max_seqlen == 0 or total_tokens == 0 enqueues nothing.
 */
size_t mimo_attn_prefill_rope_workspace_size(const mimo_attn_dims* dims, int32_t total_tokens, int32_t rotary_dim);

int mimo_attn_prefill_rope(const mimo_attn_dims* dims, int layer_type,
                           const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* positions,
                           const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen, int32_t total_tokens,
                           float rope_theta, int32_t rotary_dim, const float* sink, uint16_t* out, float* lse,
                           uint16_t* k_rot, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked prefill with the rotary embedding fused in (ABI version 12): as
 * mimo_attn_prefill_chunk (layer_type SWA or GA; pages non-NULL selects the
 * paged GA pool, else kv_base) for the chunk's un-rotated q and k, rotated as
 * mimo_attn_prefill_rope does it -- K once into k_rot by a K-only pass that
 * also writes each token's (cos, sin) table into the workspace, Q in
 * registers as the attention kernels load it -- at the caller's position ids
 * (normally ctx_lens[b] + i for token i of sequence b).  The cached keys are
 * read as they are: the caches hold post-RoPE keys (what the caller appended
 * from k_rot).  Bit-identical to mimo_rope_apply on copies of q and k
 * followed by mimo_attn_prefill_chunk(_paged) over the rotated copies.
 *
 *   positions    [total_new] int32 (device).
 *   total_new    (host) == cu_newlens[num_seqs].
 *   k_rot        [total_new][Hkv][192] bf16 (device), written; may alias k.
 *   workspace    mimo_attn_prefill_rope_workspace_size(dims, total_new,
 *                rotary_dim) bytes of device memory, scratch after the call.
 *   rope_theta, rotary_dim  as mimo_attn_prefill_rope.
 * A call with max_newlen == 0 or total_new == 0 enqueues nothing.  Other
 * errors as mimo_attn_prefill_chunk and mimo_attn_prefill_rope.
 */
int mimo_attn_prefill_chunk_rope(const mimo_attn_dims* dims, int layer_type,
                                 const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* positions,
                                 const int32_t* cu_newlens, int32_t num_seqs, int32_t max_newlen, int32_t total_new,
                                 const uint16_t* k_cache, const uint16_t* v_cache, const int64_t* kv_base,
                                 const mimo_kv_pages* pages, const int32_t* ctx_lens,
                                 float rope_theta, int32_t rotary_dim, const float* sink,
                                 uint16_t* out, float* lse, uint16_t* k_rot,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * A decode step with the rotary embedding fused in (ABI version 13; model
 * doc, MiMoV2FlashConfig: rope_parameters / rope_theta;
 * MiMoV2FlashModel.forward: position_ids, past_key_values): the outputs and
 * the caches afterwards are those of mimo_rope_apply on copies of q and k_new
 * (one token per sequence) followed by mimo_attn_decode_append over the
 * rotated copies, bit for bit, in one launch (GA: the split kernel and its
 * combine).  The queries rotate in registers as the kernels load them, the
 * new token's key where it joins the attention and again where the fused
 * append writes it, so the caches hold post-RoPE keys; each workgroup forms
 * the angles of its sequence (fp64, as mimo_rope_apply does).
 *
 * Arguments as for mimo_attn_decode_append (bf16 ring or contiguous GA pool),
 * with q and k_new before the rotation (only read), plus
 *   positions    [batch] int32 (device): the position id of sequence b's new
 *                token (normally ctx_lens[b]).
 *   rope_theta   > 1 (host).
 *   rotary_dim   a multiple of 64 in [64, 192] (host): the decode kernels hold
 *                dims 32s + 8j .. +7 of a head in one register group, so the
 *                pair (i, i + rotary_dim/2) lies in one lane for these
 *                values; others are MIMO_ERR_UNSUPPORTED (use
 *                mimo_rope_apply and mimo_attn_decode_append).
 * Errors as for mimo_attn_decode_append; NULL positions or a rope_theta that
 * is not finite and above 1 is MIMO_ERR_INVALID_ARG.
 */
int mimo_attn_decode_append_rope(const mimo_attn_dims* dims, int layer_type,
                                 const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                 const int32_t* positions, uint16_t* k_cache, uint16_t* v_cache,
                                 const int64_t* kv_base, const int64_t* kv_capacity, const int32_t* ctx_lens,
                                 int32_t batch, int32_t max_ctx, int32_t split_tokens,
                                 float rope_theta, int32_t rotary_dim, const float* sink,
                                 uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Check mode (see the conventions above).  mimo_attn_set_check switches it on
 * (enable != 0) or off for the whole process and returns the previous
 * setting; before the first call of either function the setting is
 * MIMO_ATTN_CHECK=1 from the environment.  Switching needs no device.
 */
int mimo_attn_set_check(int enable);

/*
 * Reads the current device's sticky check word into *flags (host): the OR of
 * the MIMO_CHECK_* bits of every check since the word was last cleared, on
 * any stream, captured graphs' replays included.  clear != 0 then resets it.
 * Synchronous: call it once the checked work has finished (e.g. after
 * hipDeviceSynchronize).  NULL flags is MIMO_ERR_INVALID_ARG; a HIP failure
 * is MIMO_ERR_HIP.
 */
int mimo_attn_check_flags(uint32_t* flags, int clear);

/* Static English name of a status code ("MIMO_OK", ...). */
const char* mimo_status_string(int status);

/* Message describing the calling thread's most recent non-OK return ("" if none). */
const char* mimo_last_error(void);

/* MIMO_ATTN_ABI_VERSION of the loaded library. */
int mimo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_ATTN_H */
