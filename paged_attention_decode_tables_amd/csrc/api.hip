// api.hip -- the exported C ABI of libpagedattn.so (declared in pagedattn.h).
// Every entry point validates its arguments on the host, then enqueues its
// kernels on the caller's stream. Nothing here allocates or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "kernels.h"
#include "pagedattn_probe.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int launched(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(PA_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return PA_OK;
}

int elem_size(int dtype)
{
    switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
    }
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(int64_t v)
{
    int s = 0;
    while ((int64_t(1) << s) < v) ++s;
    return s;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kMaxGridYZ = 65535;

}  // namespace

PA_EXPORT const char* pa_last_error(void) { return g_last_error.c_str(); }

namespace pa {
void set_last_error(const char* msg) { g_last_error = msg; }
}  // namespace pa

// The whole host side of paged_attn_decode: validation, parameters and the
// kernel choice. With `kind` non-null nothing is launched and the chosen
// kernel (PA_KERNEL_VALU / _MFMA / _MLA) is stored there instead.
static int decode_impl(const pa_decode_args* a, void* stream, int* kind)
{
    if (!a) return fail(PA_EINVAL, "paged_attn_decode: args is NULL");
    if (a->kernel_hint != PA_KERNEL_AUTO && a->kernel_hint != PA_KERNEL_VALU && a->kernel_hint != PA_KERNEL_MFMA)
        return fail(PA_EINVAL, "paged_attn_decode: kernel_hint %d is not PA_KERNEL_AUTO, _VALU or _MFMA", a->kernel_hint);
    const int esz = elem_size(a->dtype);
    if (!esz) return fail(PA_EINVAL, "paged_attn_decode: unknown dtype %d", a->dtype);
    const bool fp8 = a->kv_dtype == PA_FP8_E4M3;
    if (a->kv_dtype != 0 && a->kv_dtype != a->dtype && !fp8)
        return fail(PA_EINVAL, "paged_attn_decode: kv_dtype %d is neither 0, dtype nor PA_FP8_E4M3", a->kv_dtype);
    const int kv_esz = fp8 ? 1 : esz;  // cache element size
    if (fp8 && (!isfinite(a->k_scale) || !isfinite(a->v_scale) || a->k_scale == 0.0f || a->v_scale == 0.0f))
        return fail(PA_EINVAL, "paged_attn_decode: fp8 caches need finite nonzero k_scale and v_scale");
    if (a->num_seqs < 0) return fail(PA_EINVAL, "paged_attn_decode: num_seqs < 0");
    if (a->num_group < 0) return fail(PA_EINVAL, "paged_attn_decode: num_group < 0");
    const int ng = a->num_group < 1 ? 1 : a->num_group;  // query tokens per sequence
    if (a->num_heads < 1 || a->num_kv_heads < 1 || a->num_heads % a->num_kv_heads)
        return fail(PA_EINVAL, "paged_attn_decode: num_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    a->num_heads, a->num_kv_heads);
    if (a->head_size < 1 || a->v_head_size < 1)
        return fail(PA_EINVAL, "paged_attn_decode: head sizes must be positive");
    if (!pow2(a->block_size) || a->block_size > 1024)
        return fail(PA_EINVAL, "paged_attn_decode: block_size %d is not a power of two in [1, 1024]", a->block_size);
    if (a->x < 1 || a->head_size % a->x)
        return fail(PA_EINVAL, "paged_attn_decode: x = %d must divide head_size %d", a->x, a->head_size);
    if (a->x * kv_esz != 16)
        return fail(PA_ENOTSUP, "paged_attn_decode: key packing x = %d, only 16 / cache element size (%d) is built",
                    a->x, 16 / kv_esz);
    if (a->max_num_parts < 1) return fail(PA_EINVAL, "paged_attn_decode: max_num_parts < 1");
    if (a->max_seq_len < 0) return fail(PA_EINVAL, "paged_attn_decode: max_seq_len < 0");
    int64_t parts;
    const bool balanced = !a->num_splits && a->partition_size == 0;
    if (balanced) {
        if (a->num_workers < 1) return fail(PA_EINVAL, "paged_attn_decode: balanced splits need num_workers >= 1");
        if (a->max_num_parts < 2) return fail(PA_EINVAL, "paged_attn_decode: balanced splits need max_num_parts >= 2");
        parts = a->num_workers;  // grid dimension: one workgroup per token range
    } else if (!a->num_splits) {
        if (a->partition_size < 64 || a->partition_size % 64)
            return fail(PA_EINVAL, "paged_attn_decode: partition_size %d is not a positive multiple of 64", a->partition_size);
        parts = cdiv(a->max_seq_len, a->partition_size);
        if (parts > a->max_num_parts)
            return fail(PA_EINVAL, "paged_attn_decode: max_num_parts %d < cdiv(max_seq_len %d, partition_size %d) = %lld",
                        a->max_num_parts, a->max_seq_len, a->partition_size, (long long)parts);
    } else {
        parts = a->max_num_parts;
    }
    if (a->tmp_dtype != PA_F32 && a->tmp_dtype != PA_F16 && a->tmp_dtype != PA_BF16)
        return fail(PA_EINVAL, "paged_attn_decode: tmp_dtype %d is not PA_F32, PA_F16 or PA_BF16", a->tmp_dtype);
    if ((a->num_seqs == 0 || parts == 0) && !kind) return PA_OK;
    if (!a->tmp_output || !a->exp_sums || !a->max_logits || !a->query || !a->key_cache ||
        !a->value_cache || !a->block_tables || !a->seq_lens)
        return fail(PA_EINVAL, "paged_attn_decode: a required pointer is NULL");
    if (a->tmp_stride_d != 1 || a->ml_stride_p != 1 || a->q_stride_d != 1)
        return fail(PA_ENOTSUP, "paged_attn_decode: innermost strides of tmp_output, max_logits/exp_sums and query must be 1");
    const int64_t bs = a->block_size, x = a->x;
    if (a->k_stride_x != 1 || a->k_stride_bs != x || a->k_stride_dx != bs * x)
        return fail(PA_ENOTSUP, "paged_attn_decode: key_cache inner dims must be packed [head_size/x, block_size, x]");
    if (a->v_stride_bs != 1 || a->v_stride_d != bs)
        return fail(PA_ENOTSUP, "paged_attn_decode: value_cache inner dims must be packed [v_head_size, block_size]");
    // 16-byte vector accesses
    if (!aligned16(a->query) || !aligned16(a->key_cache) || !aligned16(a->value_cache) ||
        !aligned16(a->tmp_output))
        return fail(PA_ENOTSUP, "paged_attn_decode: query, caches and tmp_output must be 16-byte aligned");
    const int64_t tmp_esz = a->tmp_dtype == PA_F32 ? 4 : 2;
    if ((a->q_stride_s * esz) % 16 || (a->q_stride_h * esz) % 16 || (a->k_stride_b * kv_esz) % 16 ||
        (a->k_stride_h * kv_esz) % 16 || (a->v_stride_b * kv_esz) % 16 || (a->v_stride_h * kv_esz) % 16 ||
        (a->tmp_stride_s * tmp_esz) % 16 || (a->tmp_stride_h * tmp_esz) % 16 || (a->tmp_stride_p * tmp_esz) % 16)
        return fail(PA_ENOTSUP, "paged_attn_decode: outer strides must keep rows 16-byte aligned");
    if (parts > kMaxGridYZ || (int64_t)a->num_heads * ng > kMaxGridYZ)
        return fail(PA_ENOTSUP, "paged_attn_decode: partitions and num_heads * num_group must be <= %d", kMaxGridYZ);
    if ((int64_t)a->num_seqs * ng * a->num_heads > 0x7fffffff)
        return fail(PA_ENOTSUP, "paged_attn_decode: num_seqs * num_group * num_heads must be < 2^31");
    const int D = a->head_size, Dv = a->v_head_size, group = a->num_heads / a->num_kv_heads;
    if (!pa::decode_valu_supported(a->dtype, D, Dv))
        return fail(PA_ENOTSUP, "paged_attn_decode: (head_size, v_head_size) = (%d, %d) is not built", D, Dv);

    pa::DecodeParams p{};
    p.tmp = a->tmp_output;
    p.tmp_dtype = a->tmp_dtype;
    p.tmp_ss = a->tmp_stride_s;
    p.tmp_sh = a->tmp_stride_h;
    p.tmp_sp = a->tmp_stride_p;
    p.exp_sums = a->exp_sums;
    p.max_logits = a->max_logits;
    p.ml_ss = a->ml_stride_s;
    p.ml_sh = a->ml_stride_h;
    p.q = a->query;
    p.q_ss = a->q_stride_s;
    p.q_sh = a->q_stride_h;
    p.kc = a->key_cache;
    p.k_sb = a->k_stride_b;
    p.k_sh = a->k_stride_h;
    p.vc = a->value_cache;
    p.v_sb = a->v_stride_b;
    p.v_sh = a->v_stride_h;
    p.pl = pa::PageList{a->block_tables, a->bt_stride_s, a->bt_stride_b, a->kv_indptr};
    p.seq_lens = a->seq_lens;
    p.num_splits = a->num_splits;
    p.scale_log2 = a->scale * (fp8 ? a->k_scale : 1.0f) * pa::kLog2e;
    p.alibi = a->alibi_slopes;
    p.v_scale = fp8 ? a->v_scale : 1.0f;
    p.kv_fp8 = fp8;
    p.num_heads = a->num_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.group = group;
    p.bs_shift = log2i(bs);
    p.partition_size = a->partition_size;
    p.max_num_parts = a->max_num_parts;
    p.num_seqs = a->num_seqs;
    p.num_group = ng;
    p.num_workers = balanced ? a->num_workers : 0;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // latent rows: the value cache is the leading v_head_size columns of the key rows
    // (query-dtype or fp8 codes). The matrix-core kernels take ALiBi and fp8 caches.
    const bool mla_ok = pa::decode_mla_supported(a->dtype, D, Dv, group, a->block_size) &&
                        a->value_cache == a->key_cache && a->v_stride_b == a->k_stride_b &&
                        a->v_stride_h == a->k_stride_h;
    // its 16 columns hold the (query token, head) pairs of a kv head
    const bool mfma_ok = pa::decode_mfma_supported(a->dtype, D, Dv, group * ng, a->block_size);
    if (a->kernel_hint == PA_KERNEL_MFMA && !mfma_ok && !mla_ok)
        return fail(PA_ENOTSUP, "paged_attn_decode: no matrix-core kernel serves this problem");
    if (balanced && (!mla_ok || a->kernel_hint == PA_KERNEL_VALU))
        return fail(PA_ENOTSUP, "paged_attn_decode: balanced splits are built for the MLA matrix-core kernel only "
                                "(latent rows: V the leading columns of K, page size 1)");
    if (a->kernel_hint != PA_KERNEL_VALU && mla_ok) {
        if (kind) return *kind = PA_KERNEL_MLA, PA_OK;
        return launched(pa::launch_decode_mla(p, a->dtype, a->num_seqs, (int)parts, st),
                        "paged_attn_decode (mla)");
    }
    // Automatic choice: the matrix cores where several (query token, head)
    // columns share a kv head's rows (a real contraction), and for fp8 caches
    // also with one column. With query-dtype caches one column runs on the
    // vector ALUs: the same time on the MHA batch (78.4 us either way), so
    // the single-column tile buys nothing there; with fp8 caches the matrix
    // kernel's register-tile staging is 7% faster (46.3 vs 49.8 us).
    const bool mfma_auto = mfma_ok && (group * ng > 1 || fp8);
    if (a->kernel_hint == PA_KERNEL_MFMA ? mfma_ok : (a->kernel_hint != PA_KERNEL_VALU && mfma_auto)) {
        if (kind) return *kind = PA_KERNEL_MFMA, PA_OK;
        return launched(pa::launch_decode_mfma(p, a->dtype, D, Dv, a->num_seqs, (int)parts, st),
                        "paged_attn_decode (mfma)");
    }
    if (kind) return *kind = PA_KERNEL_VALU, PA_OK;
    return launched(pa::launch_decode_valu(p, a->dtype, D, Dv, a->num_seqs, (int)parts, st),
                    "paged_attn_decode (valu)");
}

PA_EXPORT int paged_attn_decode(const pa_decode_args* a, void* stream) { return decode_impl(a, stream, nullptr); }

PA_EXPORT int paged_attn_decode_kernel(const pa_decode_args* a)
{
    int kind = 0;
    const int rc = decode_impl(a, nullptr, &kind);
    return rc < 0 ? rc : kind;
}

PA_EXPORT int paged_attn_reduce(const pa_reduce_args* a, void* stream)
{
    if (!a) return fail(PA_EINVAL, "paged_attn_reduce: args is NULL");
    if (!elem_size(a->out_dtype)) return fail(PA_EINVAL, "paged_attn_reduce: unknown out_dtype %d", a->out_dtype);
    if (a->num_seqs < 0 || a->num_heads < 1 || a->v_head_size < 1 || a->max_num_parts < 1 || a->num_group < 0)
        return fail(PA_EINVAL, "paged_attn_reduce: num_seqs, num_group >= 0 and num_heads, v_head_size, "
                               "max_num_parts >= 1 required");
    const int ng = a->num_group < 1 ? 1 : a->num_group;
    if (!a->num_splits && a->partition_size != 0 && (a->partition_size < 64 || a->partition_size % 64))
        return fail(PA_EINVAL, "paged_attn_reduce: partition_size %d is neither 0 nor a positive multiple of 64",
                    a->partition_size);
    if (a->tmp_dtype != PA_F32 && a->tmp_dtype != PA_F16 && a->tmp_dtype != PA_BF16)
        return fail(PA_EINVAL, "paged_attn_reduce: tmp_dtype %d is not PA_F32, PA_F16 or PA_BF16", a->tmp_dtype);
    if (a->num_seqs == 0) return PA_OK;
    if (!a->output || !a->tmp_output || !a->exp_sums || !a->max_logits || !a->seq_lens)
        return fail(PA_EINVAL, "paged_attn_reduce: a required pointer is NULL");
    if (a->out_stride_d != 1 || a->tmp_stride_d != 1 || a->ml_stride_p != 1)
        return fail(PA_ENOTSUP, "paged_attn_reduce: innermost strides must be 1");
    if (!pa::reduce_supported(a->v_head_size))
        return fail(PA_ENOTSUP, "paged_attn_reduce: v_head_size %d is not built", a->v_head_size);
    const int64_t tmp_esz = a->tmp_dtype == PA_F32 ? 4 : 2;
    if (!aligned16(a->tmp_output) || (a->tmp_stride_s * tmp_esz) % 16 || (a->tmp_stride_h * tmp_esz) % 16 ||
        (a->tmp_stride_p * tmp_esz) % 16)
        return fail(PA_ENOTSUP, "paged_attn_reduce: tmp_output rows must be 16-byte aligned");
    const int64_t pairs = (int64_t)a->num_seqs * ng * a->num_heads;
    if (pairs > 0x7fffffff) return fail(PA_ENOTSUP, "paged_attn_reduce: too many (row, head) pairs");

    pa::ReduceParams p{};
    p.out = a->output;
    p.out_ss = a->out_stride_s;
    p.out_sh = a->out_stride_h;
    p.tmp = a->tmp_output;
    p.tmp_dtype = a->tmp_dtype;
    p.tmp_ss = a->tmp_stride_s;
    p.tmp_sh = a->tmp_stride_h;
    p.tmp_sp = a->tmp_stride_p;
    p.exp_sums = a->exp_sums;
    p.max_logits = a->max_logits;
    p.ml_ss = a->ml_stride_s;
    p.ml_sh = a->ml_stride_h;
    p.seq_lens = a->seq_lens;
    p.num_splits = a->num_splits;
    p.num_seqs = a->num_seqs;
    p.num_group = ng;
    p.num_heads = a->num_heads;
    p.partition_size = a->partition_size;
    p.max_num_parts = a->max_num_parts;
    return launched(pa::launch_reduce(p, a->out_dtype, a->v_head_size, reinterpret_cast<hipStream_t>(stream)),
                    "paged_attn_reduce");
}

PA_EXPORT int normal_decode_set_metadata(const pa_metadata_args* a, void* stream)
{
    if (!a) return fail(PA_EINVAL, "normal_decode_set_metadata: args is NULL");
    if (a->reserved != 0) return fail(PA_EINVAL, "normal_decode_set_metadata: reserved must be 0");
    if (a->batch < 0) return fail(PA_EINVAL, "normal_decode_set_metadata: batch < 0");
    if (a->max_seq_pages < 0) return fail(PA_EINVAL, "normal_decode_set_metadata: max_seq_pages < 0");
    if (a->page_size < 1 || (a->page_size & (a->page_size - 1)))
        return fail(PA_EINVAL, "normal_decode_set_metadata: page_size %d is not a power of two", a->page_size);
    if (!a->cu_seqlens_k) return fail(PA_EINVAL, "normal_decode_set_metadata: cu_seqlens_k is NULL");
    if (a->batch > 0 && (!a->cache_seqlens || !a->seq_lens))
        return fail(PA_EINVAL, "normal_decode_set_metadata: cache_seqlens or seq_lens is NULL");
    if (a->batch > 0 && a->max_seq_pages > 0 && (!a->page_table || !a->req_to_token || !a->req_pool_indices))
        return fail(PA_EINVAL, "normal_decode_set_metadata: page_table, req_to_token or req_pool_indices is NULL");
    const int64_t grid = pa::metadata_grid(a->batch, a->max_seq_pages);
    if (grid > 0x7fffffff)
        return fail(PA_ENOTSUP, "normal_decode_set_metadata: batch x column blocks too large (%lld workgroups)",
                    (long long)grid);
    pa::MetadataParams p{};
    p.cache_seqlens = a->cache_seqlens;
    p.cache_seqlens_stride = a->cache_seqlens_stride;
    p.cu_seqlens_k = a->cu_seqlens_k;
    p.cu_seqlens_k_stride = a->cu_seqlens_k_stride;
    p.page_table = a->page_table;
    p.page_table_stride0 = a->page_table_stride0;
    p.page_table_stride1 = a->page_table_stride1;
    const bool swa = a->swa_page_table && a->full_to_swa;
    p.swa_page_table = swa ? a->swa_page_table : nullptr;
    p.swa_page_table_stride0 = a->swa_page_table_stride0;
    p.swa_page_table_stride1 = a->swa_page_table_stride1;
    p.seq_lens = a->seq_lens;
    p.seq_lens_stride = a->seq_lens_stride;
    p.req_to_token = a->req_to_token;
    p.req_to_token_stride0 = a->req_to_token_stride0;
    p.req_to_token_stride1 = a->req_to_token_stride1;
    p.req_pool_indices = a->req_pool_indices;
    p.req_pool_indices_stride = a->req_pool_indices_stride;
    p.full_to_swa = a->full_to_swa;
    p.full_to_swa_stride = a->full_to_swa_stride;
    p.seq_len_delta = a->seq_len_delta;
    p.batch = a->batch;
    p.max_seq_pages = a->batch > 0 ? a->max_seq_pages : 0;
    int shift = 0;
    while ((1 << shift) < a->page_size) ++shift;
    p.shift = shift;
    return launched(pa::launch_decode_metadata(p, reinterpret_cast<hipStream_t>(stream)),
                    "normal_decode_set_metadata");
}

PA_EXPORT int prepare_swa_spec_page_table(int32_t* dst, int64_t dst_stride0, int64_t dst_stride1,
                                          const int32_t* page_table_a, int64_t a_stride0, int64_t a_stride1,
                                          const int32_t* page_table_b, int64_t b_stride0, int64_t b_stride1,
                                          const int32_t* seq_len_a, const int32_t* seq_len_b, int32_t bs,
                                          int32_t len_a, int32_t len_b, int32_t draft_tokens, void* stream)
{
    if (bs < 0 || len_a < 0 || len_b < 0)
        return fail(PA_EINVAL, "prepare_swa_spec_page_table: bs, len_a and len_b must be >= 0");
    if (draft_tokens < 1) return fail(PA_EINVAL, "prepare_swa_spec_page_table: draft_tokens < 1");
    if (bs == 0 || len_a + (int64_t)len_b == 0) return PA_OK;
    if (!dst || !seq_len_a || !seq_len_b || (len_a > 0 && !page_table_a) || (len_b > 0 && !page_table_b))
        return fail(PA_EINVAL, "prepare_swa_spec_page_table: a required pointer is NULL");
    const int64_t grid = pa::spec_table_grid((int64_t)bs * draft_tokens, len_a, len_b);
    if (grid > 0x7fffffff)
        return fail(PA_ENOTSUP, "prepare_swa_spec_page_table: too many rows x column blocks (%lld)",
                    (long long)grid);
    pa::SpecTableParams p{};
    p.dst = dst;
    p.dst_stride0 = dst_stride0;
    p.dst_stride1 = dst_stride1;
    p.a = page_table_a;
    p.a_stride0 = a_stride0;
    p.a_stride1 = a_stride1;
    p.b = page_table_b;
    p.b_stride0 = b_stride0;
    p.b_stride1 = b_stride1;
    p.seq_len_a = seq_len_a;
    p.seq_len_b = seq_len_b;
    p.bs = bs;
    p.len_a = len_a;
    p.len_b = len_b;
    p.draft_tokens = draft_tokens;
    return launched(pa::launch_swa_spec_page_table(p, reinterpret_cast<hipStream_t>(stream)),
                    "prepare_swa_spec_page_table");
}

PA_EXPORT int build_page_indices(int32_t* page_indices, const int32_t* block_table, int64_t bt_stride0,
                                 int64_t bt_stride1, const int32_t* cu_num_blocks, int32_t num_reqs,
                                 void* stream)
{
    if (num_reqs < 0) return fail(PA_EINVAL, "build_page_indices: num_reqs < 0");
    if (num_reqs == 0) return PA_OK;
    if (!page_indices || !block_table || !cu_num_blocks)
        return fail(PA_EINVAL, "build_page_indices: a required pointer is NULL");
    return launched(pa::launch_page_indices(page_indices, block_table, bt_stride0, bt_stride1, cu_num_blocks,
                                            num_reqs, reinterpret_cast<hipStream_t>(stream)),
                    "build_page_indices");
}

PA_EXPORT int num_kv_splits(int32_t* out, const int32_t* seq_lens, int32_t num_seq, int32_t num_group,
                            int32_t num_head, int32_t num_kv_head, int32_t max_kv_splits,
                            int32_t device_core_count, void* stream)
{
    if (num_seq < 0 || num_group < 1 || num_head < 1 || num_kv_head < 1 || max_kv_splits < 1 ||
        device_core_count < 1)
        return fail(PA_EINVAL, "num_kv_splits: num_seq >= 0 and positive group/head/split/core counts required");
    // the heuristic divides by min(16, num_head / num_kv_head)
    if (num_head < num_kv_head)
        return fail(PA_EINVAL, "num_kv_splits: num_head %d < num_kv_head %d", num_head, num_kv_head);
    if (num_seq == 0) return PA_OK;
    if (!out || !seq_lens) return fail(PA_EINVAL, "num_kv_splits: a required pointer is NULL");
    return launched(pa::launch_num_kv_splits(out, seq_lens, num_seq, num_group, num_head, num_kv_head,
                                             max_kv_splits, device_core_count,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "num_kv_splits");
}

PA_EXPORT int paged_token_offsets(int64_t* out, int64_t out_stride_s, const int32_t* block_tables,
                                  int64_t bt_stride_s, int64_t bt_stride_b, const int32_t* kv_indptr,
                                  const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                  int32_t block_size, int64_t block_stride, int64_t slot_stride,
                                  void* stream)
{
    if (num_seqs < 0 || max_seq_len < 0) return fail(PA_EINVAL, "paged_token_offsets: negative size");
    if (!pow2(block_size) || block_size > 1024)
        return fail(PA_EINVAL, "paged_token_offsets: block_size %d is not a power of two in [1, 1024]", block_size);
    if (num_seqs == 0 || max_seq_len == 0) return PA_OK;
    if (!out || !block_tables || !seq_lens) return fail(PA_EINVAL, "paged_token_offsets: a required pointer is NULL");
    if (num_seqs > kMaxGridYZ) return fail(PA_ENOTSUP, "paged_token_offsets: num_seqs > %d", kMaxGridYZ);
    pa::PageList pl{block_tables, bt_stride_s, bt_stride_b, kv_indptr};
    return launched(pa::launch_token_offsets(out, out_stride_s, pl, seq_lens, num_seqs, max_seq_len,
                                             log2i(block_size), block_stride, slot_stride,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "paged_token_offsets");
}

PA_EXPORT int pa_read_probe(const void* base0, const void* base1, const int32_t* pages, int64_t num_pages,
                            int32_t runs_per_page, int64_t page_stride, int64_t run_stride, int32_t run_bytes,
                            uint32_t* sink, int32_t workgroups, void* stream)
{
    if (num_pages < 0 || runs_per_page < 1 || workgroups < 1)
        return fail(PA_EINVAL, "pa_read_probe: num_pages >= 0, runs_per_page >= 1 and workgroups >= 1 required");
    if (run_bytes < 16 || run_bytes > 8192 || run_bytes % 16 || page_stride % 16 || run_stride % 16)
        return fail(PA_EINVAL, "pa_read_probe: run_bytes must be a multiple of 16 in [16, 8192] and the strides "
                               "multiples of 16");
    if (!sink || (num_pages > 0 && (!base0 || !pages)))
        return fail(PA_EINVAL, "pa_read_probe: a required pointer is NULL");
    if (!aligned16(base0) || !aligned16(base1) || !aligned16(sink))
        return fail(PA_EINVAL, "pa_read_probe: base0, base1 and sink must be 16-byte aligned");
    pa::ProbeParams p{};
    p.base0 = static_cast<const char*>(base0);
    p.base1 = static_cast<const char*>(base1);
    p.pages = pages;
    p.num_pages = num_pages;
    p.page_stride = page_stride;
    p.run_stride = run_stride;
    p.runs_per_page = runs_per_page;
    p.pieces = run_bytes / 16;
    p.sink = sink;
    return launched(pa::launch_read_probe(p, workgroups, reinterpret_cast<hipStream_t>(stream)), "pa_read_probe");
}
