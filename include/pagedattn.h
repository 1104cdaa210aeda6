/*
 * pagedattn.h -- C ABI of libpagedattn.so: split-KV PagedAttention decode on
 * AMD MI355X (gfx950).
 *
 * Pages the operations come from:
 *   [T2522]   triton-lang/triton issue 2522, "Needs help on performance
 *             optimization" (block-table example, index fragment).
 *   [PAv2]    paged_attention_v2_triton.py (modelhub project_6): tensor
 *             definitions in the partition- and reduce-kernel signatures,
 *             the phase-1 algorithm in the module docstring, the phase-2
 *             reduce kernel, the wrapper paged_attention_v2_triton.
 *   [PR35765] vLLM PR 35765, "AITER MLA backend: Avoid CPU sync in
 *             _build_decode" (_copy_page_indices_kernel, stride-robust form).
 *   [SGMETA]  sglang kernels/ops/attention/metadata.py
 *             (get_num_kv_splits_triton; normal_decode_set_metadata and its
 *             fused metadata kernels; prepare_swa_spec_page_table_triton).
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers (HBM of the current HIP device) unless
 *     said otherwise. The caller owns and allocates every buffer; the library
 *     allocates nothing and never synchronises with the host ([PR35765]: the
 *     point of the page-indices kernel is to avoid a host sync).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and completes asynchronously.
 *   - Strides are in ELEMENTS. Index tensors honour every stride ([PR35765]
 *     review); for the caches and activations the innermost dimensions must
 *     be packed as stated, anything else returns PA_ENOTSUP. Their base
 *     pointers and outer strides must keep every row 16-byte aligned
 *     (PA_ENOTSUP otherwise).
 *   - Return value: PA_OK (0) or a negative code. Arguments are validated on
 *     the host before any launch; an error leaves every output untouched.
 *     Values stored in device memory (lengths, block ids) cannot be checked
 *     without a host sync; the rules they must follow are stated per call.
 *     pa_last_error() returns a message for the last failure on this thread.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_EINVAL (-1)   /* bad scalar, shape, stride or null pointer */
#define PA_ENOTSUP (-2)  /* valid, but this dtype/size/layout combination is not built */
#define PA_ELAUNCH (-3)  /* the HIP launch itself failed */

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;
/* PA_FP8_E4M3 is a cache dtype only (pa_decode_args.kv_dtype). */

/*
 * Phase 1 of split-KV decode ([PAv2] _paged_attn_v2_partition_kernel and the
 * module docstring): for every sequence s, query head h and split p, over
 * the tokens t of split p:
 *     z_t = scale * q[s,h,:] . K_t,   m = max_t z_t,   l = sum_t exp(z_t - m),
 *     tmp = sum_t exp(z_t - m) V_t / l
 * and stores max_logits[s,h,p] = m, exp_sums[s,h,p] = l, tmp_output[s,h,p,:]
 * = tmp (the normalised split output; phase 2 weights it by exp(m - M) * l).
 * Query head h reads kv head h / (num_heads / num_kv_heads).
 *
 * Token t of sequence s is gathered in two steps ([PAv2] docstring; [T2522]):
 * block = pages[t / block_size], slot = t % block_size, then
 *     K_t[d] = key_cache[block, kvh, d / x, slot, d % x]
 *     V_t[d] = value_cache[block, kvh, d, slot].
 *
 * Splits: with num_splits == NULL, split p covers [p*P, min((p+1)*P, L))
 * with P = partition_size ([PAv2]: PARTITION_SIZE = 512). With a num_splits
 * array (e.g. from num_kv_splits()), n_s = clamp(num_splits[s], 1,
 * max_num_parts), the split length is cdiv(L, n_s) rounded up to a multiple
 * of 64 tokens, and split p covers [p*len, min((p+1)*len, L)). A split with
 * no tokens (p*len >= L) stores m = -inf, l = 0 and leaves tmp_output
 * untouched, as the page's early exit does.
 *
 * Balanced splits (partition_size == 0, num_splits == NULL, num_workers >= 1;
 * served by the MLA matrix-core kernel only, PA_ENOTSUP otherwise): the
 * tokens of all sequences in sequence order, each sequence with L_s >= 1
 * preceded by C = 256 virtual tokens (the cost of starting a split), total
 * T' = sum over L_s >= 1 of (L_s + C), are cut into ranges of U positions,
 *     U = round_up(max(cdiv(T', num_workers), cdiv(max_s L_s, max_num_parts - 1)), 32),
 * range w = [w*U, (w+1)*U). Token t of sequence s sits at position
 * V_s + C + t, V_s = sum over earlier sequences with L >= 1 of (L + C). The
 * k-th range that meets sequence s's tokens is its split k, and slots k >=
 * (number of such ranges) store m = -inf, l = 0. So every worker gets the
 * same amount of work, counting the splits it starts, whatever the length
 * mix, and a sequence never has more than max_num_parts splits
 * (max_num_parts >= 2).
 * The live slots of a sequence are always a prefix (slots 0 .. k_max).
 * Phase 2 with partition_size == 0 merges the slots before the first one
 * whose max is -inf; the final output is the same as with any other split.
 *
 * Query groups (num_group = g > 1; [SGMETA] get_num_kv_splits_triton's
 * num_group, its output indexed seq * num_group + group): each sequence has g
 * query tokens, and every one of them attends over the sequence's whole
 * cache (the pages define no masks among them). query, tmp_output,
 * max_logits, exp_sums and output then have num_seqs * g rows, row s * g + j
 * for token j of sequence s; seq_lens and the page lists stay per sequence;
 * num_splits, when given, has num_seqs * g entries, and the g entries of a
 * sequence must be equal (num_kv_splits writes them so). The grouped-head
 * matrix-core kernel serves the g tokens of a kv head together (g * G <= 16
 * columns), reading each K/V byte once for all of them.
 *
 * Variants of phase 1 named by the [PAv2] wrapper arguments (alibi_slopes,
 * kv_cache_dtype, k_scale, v_scale), whose math the page does not give; the
 * readings implemented:
 *   ALiBi: with alibi_slopes (fp32 [num_heads]) each score gets
 *     slope[h] * (t - (L - 1)), t the token's position in its sequence of
 *     length L (the query is the last position).
 *   fp8 cache: with kv_dtype = PA_FP8_E4M3 both caches hold OCP FP8 E4M3
 *     codes (sign, 4-bit exponent with bias 7, 3-bit mantissa, no
 *     infinities, NaN = exponent 15 and mantissa 7), packed with x = 16, and
 *     K_t[d] = E4M3(code) * k_scale, V_t[d] = E4M3(code) * v_scale. The query
 *     (and every output) keeps dtype.
 */
typedef struct pa_decode_args {
    /* outputs: workspaces (tmp_output of tmp_dtype, the statistics fp32) */
    void* tmp_output;            /* [num_seqs, num_heads, max_num_parts, v_head_size] */
    int64_t tmp_stride_s, tmp_stride_h, tmp_stride_p, tmp_stride_d; /* stride_d must be 1 */
    float* exp_sums;             /* [num_seqs, num_heads, max_num_parts] */
    float* max_logits;           /* same shape and strides as exp_sums */
    int64_t ml_stride_s, ml_stride_h, ml_stride_p;                  /* stride_p must be 1 */

    /* inputs, all of element type `dtype` */
    const void* query;           /* [num_seqs, num_heads, head_size] */
    int64_t q_stride_s, q_stride_h, q_stride_d;                     /* stride_d must be 1 */
    const void* key_cache;       /* [num_blocks, num_kv_heads, head_size/x, block_size, x] */
    int64_t k_stride_b, k_stride_h, k_stride_dx, k_stride_bs, k_stride_x;
                                 /* dx, bs, x must be block_size*x, x, 1 */
    const void* value_cache;     /* [num_blocks, num_kv_heads, v_head_size, block_size] */
    int64_t v_stride_b, v_stride_h, v_stride_d, v_stride_bs;
                                 /* d, bs must be block_size, 1. value_cache may alias
                                    key_cache (MLA-style latent rows with block_size 1,
                                    V = the first v_head_size values of each row). */

    /* page lists (int32 physical block ids):
       kv_indptr == NULL: pages = block_tables[num_seqs, max_blocks] with strides
         (bt_stride_s, bt_stride_b);
       kv_indptr != NULL: CSR form ([PR35765] paged_kv_indptr/paged_kv_indices):
         the pages of sequence s are block_tables[(kv_indptr[s] + i) * bt_stride_b].
       Sequence s must list at least cdiv(seq_lens[s], block_size) valid block
       ids in [0, num_blocks); entries past that are never read. */
    const int32_t* block_tables;
    int64_t bt_stride_s, bt_stride_b;
    const int32_t* kv_indptr;    /* optional, [num_seqs + 1] */
    const int32_t* seq_lens;     /* [num_seqs]; each must be <= max_seq_len. L <= 0 gives
                                    only empty splits. */
    const int32_t* num_splits;   /* optional, [num_seqs] (see "Splits" above) */

    float scale;                 /* multiplies q . k before the softmax */
    int32_t num_seqs, num_heads, num_kv_heads;
    int32_t head_size;           /* D  */
    int32_t v_head_size;         /* Dv */
    int32_t block_size;          /* power of two, 1..1024 */
    int32_t x;                   /* key packing: 16 / element size ([PAv2] X_PACK) */
    int32_t partition_size;      /* > 0 and a multiple of 64 when num_splits == NULL */
    int32_t max_num_parts;       /* partition dimension of the workspaces; must be
                                    >= cdiv(max_seq_len, partition_size) without num_splits */
    int32_t max_seq_len;         /* host-side bound on seq_lens (sizes the grid) */
    int32_t dtype;               /* pa_dtype of query, key_cache and value_cache */
    int32_t kernel_hint;         /* PA_KERNEL_AUTO (0): pick the kernel; PA_KERNEL_VALU: the
                                    vector-ALU kernel; PA_KERNEL_MFMA: the matrix-core kernel
                                    (PA_ENOTSUP where it does not apply); any other value
                                    is PA_EINVAL. Results agree within the documented
                                    tolerance either way. */
    int32_t num_workers;         /* balanced splits only (partition_size == 0): number of
                                    token ranges. One range per workgroup: one
                                    workgroup fills a compute unit at 128 heads per
                                    kv head, two share one at 64 heads, so the
                                    compute-unit count or twice it. Ignored
                                    otherwise */
    const float* alibi_slopes;   /* optional, [num_heads] fp32 (see "Variants") */
    int32_t kv_dtype;            /* 0 (or equal to dtype): caches hold dtype;
                                    PA_FP8_E4M3: fp8 caches with the scales below */
    float k_scale, v_scale;      /* fp8 caches only; must be finite and nonzero */
    int32_t num_group;           /* query tokens per sequence (0 or 1: one); see
                                    "Query groups" */
    int32_t tmp_dtype;           /* element type of tmp_output: PA_F32 (0, the default),
                                    PA_F16 or PA_BF16. [PAv2] phase 1 stores the split
                                    output converted to the workspace's element type;
                                    16-bit types are rounded to nearest even, which
                                    halves the workspace traffic of both phases. */
} pa_decode_args;

#define PA_KERNEL_AUTO 0
#define PA_KERNEL_VALU 1
#define PA_KERNEL_MFMA 2
#define PA_KERNEL_MLA 3  /* returned by paged_attn_decode_kernel only; not a hint */

/*
 * Supported combinations (others return PA_ENOTSUP):
 *   dtype f32, f16, bf16 with x = 16 / element size;
 *   (head_size, v_head_size) in {(64,64), (128,128), (256,256), (576,512)};
 *   any group size num_heads / num_kv_heads.
 * Kernel choice (PA_KERNEL_AUTO): latent rows (D = 576, Dv = 512, page size
 * 1, value_cache = key_cache, 64 or 128 heads a kv head, f16/bf16 queries)
 * on the latent-row matrix-core kernel, with query-dtype or fp8 caches and
 * fixed or balanced splits; f16/bf16 queries with D = Dv in {64, 128},
 * block_size >= 8 and num_group * group in 2..16 (or 1 with fp8 caches) on
 * the grouped-head matrix-core kernel; everything else on the vector
 * kernel. PA_KERNEL_MFMA also takes one column with query-dtype caches.
 * ALiBi slopes and fp8 caches (x = 16) run on every kernel. Balanced splits
 * need the latent-row kernel (PA_ENOTSUP otherwise).
 */
int paged_attn_decode(const pa_decode_args* args, void* stream);

/*
 * The phase-1 kernel paged_attn_decode would launch for `args`
 * (PA_KERNEL_VALU: the vector kernel, PA_KERNEL_MFMA: the grouped-head
 * matrix-core kernel, PA_KERNEL_MLA: the latent-row kernel), after the same
 * validation and with the same error codes, or a negative error. Host only:
 * nothing is launched or read through the pointers, which must still pass
 * the checks (non-null, aligned). An empty batch reports the kernel too.
 */
int paged_attn_decode_kernel(const pa_decode_args* args);

/*
 * Phase 2 ([PAv2] _paged_attn_v2_reduce_kernel): for each (s, h), over the n
 * nonempty splits of sequence s (the split rule of paged_attn_decode),
 *     M = max_p m_p,  w_p = exp(m_p - M) * l_p,
 *     output[s,h,:] = sum_p w_p * tmp_output[s,h,p,:] / sum_p w_p.
 * Every split is merged (no cap on the number of partitions). Splits past n
 * are never read, so their workspace contents do not matter. A sequence with
 * L <= 0 gets a zero output row.
 */
typedef struct pa_reduce_args {
    void* output;                /* [num_seqs, num_heads, v_head_size] of out_dtype */
    int64_t out_stride_s, out_stride_h, out_stride_d;               /* stride_d must be 1 */
    int32_t out_dtype;           /* pa_dtype */
    const void* tmp_output;      /* of tmp_dtype, as written by paged_attn_decode */
    int64_t tmp_stride_s, tmp_stride_h, tmp_stride_p, tmp_stride_d; /* stride_d must be 1 */
    const float* exp_sums;
    const float* max_logits;
    int64_t ml_stride_s, ml_stride_h, ml_stride_p;                  /* stride_p must be 1 */
    const int32_t* seq_lens;     /* [num_seqs] */
    const int32_t* num_splits;   /* optional, as given to paged_attn_decode */
    int32_t num_seqs, num_heads, v_head_size;
    int32_t partition_size;      /* as given to paged_attn_decode; 0 = balanced splits:
                                    merge the slots before the first one whose
                                    max_logits is -inf */
    int32_t max_num_parts;
    int32_t num_group;           /* as given to paged_attn_decode: output, tmp_output,
                                    max_logits and exp_sums have num_seqs * num_group rows */
    int32_t tmp_dtype;           /* as given to paged_attn_decode (0: PA_F32); the merge
                                    itself runs in fp32 */
} pa_reduce_args;

int paged_attn_reduce(const pa_reduce_args* args, void* stream);

/*
 * Flat page list from a block table ([PR35765] _copy_page_indices_kernel,
 * stride-robust form from its review): for each request r,
 *     page_indices[cu_num_blocks[r] + i] = block_table[r*bt_stride0 + i*bt_stride1]
 * for 0 <= i < cu_num_blocks[r+1] - cu_num_blocks[r]. cu_num_blocks is an
 * int32 indptr of num_reqs + 1 entries, non-decreasing, with row r holding at
 * least cu[r+1] - cu[r] entries; page_indices holds cu[num_reqs] entries.
 * num_reqs == 0 is a no-op.
 */
int build_page_indices(int32_t* page_indices, const int32_t* block_table, int64_t bt_stride0,
                       int64_t bt_stride1, const int32_t* cu_num_blocks, int32_t num_reqs,
                       void* stream);

/*
 * Split-count heuristic ([SGMETA] get_num_kv_splits_triton), one workgroup,
 * no host sync. With max and min of the lengths (a length <= 0 counts as 1):
 * if max*8 < min*10 then min = max; chunk_1 = cdiv(max, min(cdiv(max, min),
 * max_kv_splits)); cores_ext = int32(fp32(cores) * max(log2(fp32(max)/64), 1))
 * in fp32 with log2 correctly rounded to fp32; with group = num_head /
 * num_kv_head the token grid is num_seq*num_group*num_head (group 1) or
 * num_seq*num_group*cdiv(num_head, min(16, group)); chunk_2 = cdiv(max,
 * min(cdiv(cores_ext, grid), max_kv_splits)); and
 *     out[s*num_group + g] = max(cdiv(L_s, chunk_1), cdiv(L_s, chunk_2)).
 * out holds num_seq * num_group int32 entries. num_seq == 0 is a no-op.
 * PA_EINVAL for num_head < num_kv_head (a group size of 0) and for counts
 * below 1.
 */
int num_kv_splits(int32_t* out, const int32_t* seq_lens, int32_t num_seq, int32_t num_group,
                  int32_t num_head, int32_t num_kv_head, int32_t max_kv_splits,
                  int32_t device_core_count, void* stream);

/*
 * Test hook for the token -> (block, slot) map ([T2522] block-table
 * example). It runs the device functions every decode kernel uses to look
 * up a token's block and (block sizes above 1) its slot, page_of and
 * slot_of in csrc/common.h: for t < seq_lens[s],
 *     out[s*out_stride_s + t] = pages[t / block_size] * block_stride
 *                              + (t % block_size) * slot_stride
 * with the page list as in pa_decode_args (kv_indptr may be NULL). Entries
 * t >= seq_lens[s] are not written; out rows must hold max_seq_len entries.
 */
int paged_token_offsets(int64_t* out, int64_t out_stride_s, const int32_t* block_tables,
                        int64_t bt_stride_s, int64_t bt_stride_b, const int32_t* kv_indptr,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                        int32_t block_size, int64_t block_stride, int64_t slot_stride,
                        void* stream);

/*
 * Decode metadata, the step before the path ([SGMETA]
 * normal_decode_set_metadata; the five steps of its docstring, the index
 * arithmetic of its two fused kernels), in one launch:
 *   cache_seqlens[b] = int32(seq_lens[b] + seq_len_delta)
 *   cu_seqlens_k[b]  = cache_seqlens[0] + ... + cache_seqlens[b-1]  (b <= B)
 *   slot             = req_to_token[req_pool_indices[b], col * page_size]
 *   page_table[b, col]     = floor(slot / page_size)
 *   swa_page_table[b, col] = floor(full_to_swa[slot] / page_size)   (optional)
 * for 0 <= b < batch and 0 <= col < max_seq_pages. Every column below
 * max_seq_pages is written for every row, whatever the row's length.
 *
 * Types and layout: seq_lens and req_pool_indices int64; req_to_token,
 * full_to_swa and every output int32; all arrays strided in elements (any
 * stride values). int32 results wrap in two's complement (the lengths are
 * the low 32 bits of the int64 sum; the prefix sum runs in int32). Slots are
 * divided with an arithmetic right shift by log2(page_size), i.e. toward
 * minus infinity.
 *
 * page_size must be a power of two >= 1, batch >= 0, max_seq_pages >= 0
 * (PA_EINVAL otherwise). cu_seqlens_k (batch + 1 entries) is always written,
 * cu_seqlens_k[0] = 0 even for an empty batch. The SWA table is built only
 * when both swa_page_table and full_to_swa are non-NULL. Device-side values
 * must index inside the caller's arrays: req_pool_indices[b] a row of
 * req_to_token, which holds at least (max_seq_pages - 1) * page_size + 1
 * columns; every gathered slot an entry of full_to_swa when it is given.
 */
typedef struct pa_metadata_args {
    int32_t* cache_seqlens;      /* [batch] */
    int64_t cache_seqlens_stride;
    int32_t* cu_seqlens_k;       /* [batch + 1] */
    int64_t cu_seqlens_k_stride;
    int32_t* page_table;         /* [batch, max_seq_pages] */
    int64_t page_table_stride0, page_table_stride1;
    int32_t* swa_page_table;     /* [batch, max_seq_pages] or NULL */
    int64_t swa_page_table_stride0, swa_page_table_stride1;
    const int64_t* seq_lens;     /* [batch] */
    int64_t seq_lens_stride;
    const int32_t* req_to_token; /* [pool rows, context] token slots */
    int64_t req_to_token_stride0, req_to_token_stride1;
    const int64_t* req_pool_indices; /* [batch] row of req_to_token per request */
    int64_t req_pool_indices_stride;
    const int32_t* full_to_swa;  /* [slots] full-pool slot -> SWA slot, or NULL */
    int64_t full_to_swa_stride;
    int32_t batch;
    int32_t max_seq_pages;
    int32_t page_size;
    int32_t reserved;            /* must be 0 */
    int64_t seq_len_delta;
} pa_metadata_args;

int normal_decode_set_metadata(const pa_metadata_args* args, void* stream);

/*
 * Speculative SWA page table ([SGMETA] prepare_swa_spec_page_table_triton
 * and its kernel): concatenates each request's page table with the
 * expanded page tables of its draft rows. With R = draft_tokens, row m of
 * dst (0 <= m < bs*R) belongs to request m / R; with la = seq_len_a[m / R],
 * lb = seq_len_b[m], for n < min(la + lb, len_a + len_b):
 *     dst[m, n] = page_table_a[m / R, n]   if n < la  (0 if n >= len_a)
 *                 page_table_b[m, n - la]  otherwise (0 if n - la >= len_b)
 * Columns n >= la + lb are not written. Shapes: page_table_a [bs, len_a],
 * page_table_b [bs*R, len_b], dst [bs*R, len_a + len_b], seq_len_a [bs],
 * seq_len_b [bs*R]; int32 throughout, element strides. Reads are masked by
 * the table widths and writes by the destination width, so any length
 * values are memory-safe. bs, len_a, len_b >= 0 and draft_tokens >= 1
 * (PA_EINVAL otherwise); bs == 0 or len_a + len_b == 0 is a no-op.
 */
int prepare_swa_spec_page_table(int32_t* dst, int64_t dst_stride0, int64_t dst_stride1,
                                const int32_t* page_table_a, int64_t a_stride0, int64_t a_stride1,
                                const int32_t* page_table_b, int64_t b_stride0, int64_t b_stride1,
                                const int32_t* seq_len_a, const int32_t* seq_len_b, int32_t bs,
                                int32_t len_a, int32_t len_b, int32_t draft_tokens, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * paged_attn_decode() followed by paged_attn_reduce() in one call, with the
 * split partials (tmp_output, max_logits, exp_sums) in a scratch buffer the
 * library holds in device memory, PA_STATIC_SCRATCH_BYTES per GPU, from the
 * first load of its code on that GPU until the process ends. Nothing is
 * allocated per call.
 *
 * args is as for paged_attn_decode() except that tmp_output, exp_sums and
 * max_logits must be NULL (their strides are ignored); max_num_parts sizes
 * the partials, which need num_seqs * max(num_group, 1) * num_heads *
 * max_num_parts * (v_head_size * e + 8) bytes, e = 4 for tmp_dtype PA_F32
 * and 2 for PA_F16 / PA_BF16. More than PA_STATIC_SCRATCH_BYTES returns
 * PA_EINVAL before any work is queued.
 * output [num_seqs * max(num_group, 1), num_heads, v_head_size] of out_dtype
 * (f32, f16 or bf16), row strides out_stride_s, out_stride_h, innermost
 * stride 1, receives the merged result of paged_attn_reduce().
 *
 * Every call on one GPU shares that GPU's buffer and leaves its partials in
 * it; nothing in it needs to start at zero (phase 1 writes every statistic
 * phase 2 reads). Calls that overlap in time on one GPU (other streams,
 * other host threads) race on the buffer: the caller must order them.
 */
#define PA_STATIC_SCRATCH_BYTES (256u << 20)
int paged_attn_decode_static(const pa_decode_args* args, void* output, int64_t out_stride_s,
                             int64_t out_stride_h, int32_t out_dtype, void* stream);

/* Message describing the last non-OK return on the calling thread. */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
