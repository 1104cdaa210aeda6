/*
 * oracle.c -- plain, slow, obviously correct CPU reference for split-KV
 * PagedAttention decode and its two integer helpers.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. It shares no
 * code, header, table or helper with the GPU library, and the GPU library
 * never loads it.
 *
 * Sources (the web pages the method comes from):
 *   [T2522]  triton-lang/triton issue 2522, "Needs help on performance
 *            optimization": the block-table example (block table [40, 30],
 *            block size 8 -> token offsets 40..47 then 30..37) and the kernel
 *            fragment that forms block_idx * stride_kb + offs * stride_kbs.
 *   [PAv2]   paged_attention_v2_triton.py (modelhub project_6): the tensor
 *            definitions in the two kernel signatures, the phase-1 algorithm
 *            (module docstring and the commented gather steps inside the
 *            partition kernel) and the complete phase-2 reduce kernel.
 *   [PR35765] vLLM PR 35765, "AITER MLA backend: Avoid CPU sync in
 *            _build_decode": _copy_page_indices_kernel and the review's
 *            stride-robust version of it.
 *   [SGMETA] sglang kernels/ops/attention/metadata.py:
 *            get_num_kv_splits_triton, normal_decode_set_metadata with its
 *            two fused metadata kernels (the docstring lists the five steps;
 *            the kernels fix the index arithmetic), and the speculative SWA
 *            page-table concat (prepare_swa_spec_page_table_triton and its
 *            kernel).
 *
 * Precision: attention is accumulated in double. The split heuristic follows
 * the fp32 arithmetic its page prescribes (tl.float32 cast, fp32 log2 and
 * multiply, truncating cast back to int32).
 *
 * Readings where the pages are silent (each one is listed in the design notes
 * of the repository as well):
 *   R1  phase 1 stores the per-partition NORMALISED output acc / l, because
 *       the phase-2 kernel of [PAv2] weights each partition's output by
 *       exp(m_p - M) * l_p / sum, which is only right for normalised rows.
 *   R2  query head h reads kv head h / (H / Hkv) (the [PAv2] code leaves the
 *       GQA map as a TODO placeholder).
 *   R3  a sequence of length <= 0 yields an all-zero output row and only
 *       empty partitions.
 *   R4  with a per-sequence split count n_s (as produced by the heuristic of
 *       [SGMETA]), n_s is clamped to [1, max_num_parts], the split length is
 *       cdiv(L, n_s) rounded up to a multiple of 64 tokens, and split j covers
 *       [j*len, min((j+1)*len, L)). With a fixed partition size P the split
 *       length is P ([PAv2]: part_start = part_idx * PARTITION_SIZE).
 *   R5  the heuristic treats a length <= 0 as 1 (its page would divide by a
 *       zero minimum length).
 *   R6  decode metadata: seq_lens and req_pool_indices are int64 (the
 *       docstring casts seq_lens from int64; the pool indices are taken to
 *       be the same index type); req_to_token, the SWA map and every output
 *       are int32.
 *   R7  int32 results wrap in two's complement: cache_seqlens is the low 32
 *       bits of seq_len + delta and the prefix sum runs in int32.
 *   R8  the page table is gathered for every column below max_seq_pages of
 *       every row, whatever that row's length (the kernels mask on
 *       max_seq_pages only).
 *   R9  page = slot floor-divided by the page size (the docstring's floor
 *       division; the kernels' arithmetic right shift by log2(page size) is
 *       the same thing for a power-of-two size, negative slots included).
 *   R10 with an empty batch, cu_seqlens_k[0] = 0 is still written (the
 *       prefix sum of nothing).
 *   R11 the SWA table is built only when both it and the full-to-SWA map are
 *       given; it maps the raw slot (before the division) and then divides.
 *   R13 ALiBi ([PAv2] wrapper argument alibi_slopes, no math on the page):
 *       the standard linear bias, z_t = scale * q . K_t + slope[h] * (t - (L-1))
 *       with t the token's position in its sequence of length L (the query is
 *       the last position, so its own token gets no bias and earlier ones a
 *       penalty growing with the distance, for a positive slope).
 *   R14 fp8 cache ([PAv2] wrapper arguments kv_cache_dtype, k_scale, v_scale,
 *       no math on the page): both caches hold OCP FP8 E4M3 codes, packed with
 *       x = 16 (16 / element size, as for every dtype), and the dequantized
 *       values are K_t[d] = e4m3(code) * k_scale, V_t[d] = e4m3(code) *
 *       v_scale; the query keeps its own dtype.
 *   R15 e4m3(code): sign bit, 4-bit exponent e (bias 7), 3-bit mantissa m:
 *       e = 0 gives m * 2^-9, e = 15 with m = 7 is NaN, otherwise
 *       (1 + m/8) * 2^(e-7) (the OCP E4M3 definition: no infinities).
 *   R12 speculative SWA page table: the destination has LEN_A + LEN_B columns
 *       (the wrapper's LEN_OUT) and only columns below
 *       min(seq_len_a + seq_len_b, LEN_A + LEN_B) are written (the page's
 *       grid would write to the end of the last 256-column block when the
 *       lengths exceed the tables); lengths are int32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* Planted-mistake switch for the pin tests: each nonzero value builds a
 * deliberately wrong variant so the tests can show the pins catch it. The
 * default build (ORACLE_MUTANT undefined or 0) is the real oracle. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

static int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

/* Physical block holding logical block `logical` of sequence s. The page list
 * is either a 2-D block table (row s at s * stride_s) or, when indptr is
 * given, a flat CSR list whose row s starts at indptr[s] ([PR35765]:
 * paged_kv_indptr / paged_kv_indices). Elements are stride_b apart. */
static int64_t physical_block(const int32_t* pages, int64_t stride_s, int64_t stride_b,
                              const int32_t* indptr, int s, int64_t logical)
{
    int64_t row = indptr ? (int64_t)indptr[s] : (int64_t)s * stride_s;
    return (int64_t)pages[row + logical * stride_b];
}

/* ------------------------------------------------------------------------
 * Token -> cache offset map. [T2522] block-table example and fragment:
 * token t of a sequence lives in physical block bt[t / block_size] at slot
 * t % block_size, and its offset is that block times the block stride plus
 * the slot times the slot stride. Positions t >= seq_len are not written.
 * ------------------------------------------------------------------------ */
int orc_token_offsets(int64_t* out, int64_t out_stride_s,
                      const int32_t* pages, int64_t pg_stride_s, int64_t pg_stride_b,
                      const int32_t* indptr, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t block_size, int64_t block_stride, int64_t slot_stride)
{
    if (!out || !pages || !seq_lens || num_seqs < 0 || block_size < 1) return ORC_EINVAL;
    for (int s = 0; s < num_seqs; ++s) {
        for (int64_t t = 0; t < seq_lens[s]; ++t) {
            int64_t logical = t / block_size;
            int64_t slot = t % block_size;
#if ORACLE_MUTANT == 1
            slot = (t + 1) % block_size; /* planted: off-by-one slot */
#endif
            int64_t blk = physical_block(pages, pg_stride_s, pg_stride_b, indptr, s, logical);
            out[(int64_t)s * out_stride_s + t] = blk * block_stride + slot * slot_stride;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Flat page list from a block table and an indptr. [PR35765]
 * _copy_page_indices_kernel (stride-robust form from the review): for request
 * r, page_indices[cu[r] + i] = block_table[r, i] for 0 <= i < cu[r+1] - cu[r],
 * the row read with both of its strides.
 * ------------------------------------------------------------------------ */
int orc_page_indices(int32_t* page_indices, const int32_t* block_table,
                     int64_t stride0, int64_t stride1, const int32_t* cu_num_blocks,
                     int32_t num_reqs)
{
    if (num_reqs < 0) return ORC_EINVAL;
    if (num_reqs == 0) return ORC_OK;
    if (!page_indices || !block_table || !cu_num_blocks) return ORC_EINVAL;
    for (int r = 0; r < num_reqs; ++r) {
        int64_t start = cu_num_blocks[r];
        int64_t n = (int64_t)cu_num_blocks[r + 1] - start;
        for (int64_t i = 0; i < n; ++i) {
#if ORACLE_MUTANT == 2
            page_indices[start + i] = block_table[(int64_t)r * stride0 + i]; /* planted: ignores stride1 */
#else
            page_indices[start + i] = block_table[(int64_t)r * stride0 + i * stride1];
#endif
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Split-count heuristic, [SGMETA] get_num_kv_splits_triton, in the page's
 * order:
 *   max and min sequence length; if max*8 < min*10 the min is taken to be
 *   the max; splits_1 = min(cdiv(max, min), max_kv_splits) and
 *   chunk_1 = cdiv(max, splits_1);
 *   ext = fp32(max) / 64; cores_ext = int32(cores * max(log2(ext), 1));
 *   with group = num_head / num_kv_head, the token grid is
 *   num_seq*num_group*num_head for group 1, else
 *   num_seq*num_group*cdiv(num_head, min(16, group));
 *   splits_2 = min(cdiv(cores_ext, grid), max_kv_splits) and
 *   chunk_2 = cdiv(max, splits_2);
 *   n_s = max(cdiv(L_s, chunk_1), cdiv(L_s, chunk_2)), stored for each of the
 *   num_group query groups at index s*num_group + g.
 * log2 is taken as the double log2 rounded to fp32 (the page's fp32 log2,
 * correctly rounded), and the product is one fp32 multiply.
 * ------------------------------------------------------------------------ */
int orc_num_kv_splits(int32_t* out, const int32_t* seq_lens, int32_t num_seq,
                      int32_t num_group, int32_t num_head, int32_t num_kv_head,
                      int32_t max_kv_splits, int32_t device_core_count)
{
    if (num_seq < 0 || num_group < 1 || num_head < 1 || num_kv_head < 1 ||
        max_kv_splits < 1 || device_core_count < 1)
        return ORC_EINVAL;
    if (num_seq == 0) return ORC_OK;
    if (!out || !seq_lens) return ORC_EINVAL;

    int64_t max_len = 0, min_len = 0;
    for (int s = 0; s < num_seq; ++s) {
        int64_t L = seq_lens[s] < 1 ? 1 : seq_lens[s]; /* R5 */
        if (s == 0 || L > max_len) max_len = L;
        if (s == 0 || L < min_len) min_len = L;
    }
#if ORACLE_MUTANT == 3
    if (max_len * 10 < min_len * 8) min_len = max_len; /* planted: rule reversed */
#else
    if (max_len * 8 < min_len * 10) min_len = max_len;
#endif
    int64_t splits1 = min64(cdiv64(max_len, min_len), max_kv_splits);
    int64_t chunk1 = cdiv64(max_len, splits1);

    float ext = (float)max_len / 64.0f;
    float lg = (float)log2((double)ext);
#if ORACLE_MUTANT == 4
    float f = (float)device_core_count * lg; /* planted: log2 not clamped at 1 */
    if (f < 1.0f) f = 1.0f;
#else
    float f = (float)device_core_count * fmaxf(lg, 1.0f);
#endif
    int64_t cores_ext = (int64_t)(int32_t)f;

    int64_t group = num_head / num_kv_head;
    int64_t grid;
    if (group == 1)
        grid = (int64_t)num_seq * num_group * num_head;
    else
        grid = (int64_t)num_seq * num_group * cdiv64(num_head, min64(16, group));
    int64_t splits2 = min64(cdiv64(cores_ext, grid), max_kv_splits);
    int64_t chunk2 = cdiv64(max_len, splits2);

    for (int s = 0; s < num_seq; ++s) {
        int64_t L = seq_lens[s] < 1 ? 1 : seq_lens[s];
        int64_t n = max64(cdiv64(L, chunk1), cdiv64(L, chunk2));
        for (int g = 0; g < num_group; ++g) out[(int64_t)s * num_group + g] = (int32_t)n;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Attention over paged caches.
 *
 * Layouts ([PAv2] kernel signatures), element strides given for the outer
 * dims, inner dims packed:
 *   query       [S, H, D]                 (q_s, q_h, 1)
 *   key_cache   [NB, Hkv, D/x, bs, x]     (k_b, k_h, bs*x, x, 1)
 *   value_cache [NB, Hkv, Dv, bs]         (v_b, v_h, bs, 1)
 * The two-step gather ([PAv2] docstring): the physical block is
 * block_tables[s, t / bs], then K row t is key_cache[block, kvh, :, t % bs, :]
 * read as D consecutive values, and V row t is value_cache[block, kvh, :, t % bs].
 * ------------------------------------------------------------------------ */
typedef struct {
    const float* query; int64_t q_s, q_h;
    const float* key_cache; int64_t k_b, k_h;
    const float* value_cache; int64_t v_b, v_h;
    const int32_t* pages; int64_t pg_s, pg_b;
    const int32_t* indptr;
    const int32_t* seq_lens;
    int32_t S, H, Hkv, D, Dv, bs, x;
    double scale;
    /* R13, R14: optional ALiBi slopes [H]; fp8 caches (codes addressed with
       the same strides as the float caches, which are then unused) */
    const float* alibi;
    const uint8_t* key_u8;
    const uint8_t* value_u8;
    double k_scale, v_scale;
} orc_problem;

/* R15: OCP FP8 E4M3 code -> value */
static double e4m3(uint8_t c)
{
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
#if ORACLE_MUTANT == 18
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -10);              /* planted: exponent bias 8 */
    else v = ldexp(1.0 + m / 8.0, e - 8);
#else
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
#endif
    return sgn ? -v : v;
}

static int kv_head_of(const orc_problem* p, int h)
{
#if ORACLE_MUTANT == 5
    return h % p->Hkv; /* planted: interleaved GQA map */
#else
    return h / (p->H / p->Hkv); /* R2 */
#endif
}

/* Gather K rows [L][D] and V rows [L][Dv] of (s, kvh) into contiguous doubles. */
static void gather_seq(const orc_problem* p, int s, int kvh, int64_t L, double* K, double* V)
{
    for (int64_t t = 0; t < L; ++t) {
        int64_t blk = physical_block(p->pages, p->pg_s, p->pg_b, p->indptr, s, t / p->bs);
        int64_t slot = t % p->bs;
        const int64_t kbase = blk * p->k_b + (int64_t)kvh * p->k_h;
        const int64_t vbase = blk * p->v_b + (int64_t)kvh * p->v_h;
        for (int d = 0; d < p->D; ++d) {
#if ORACLE_MUTANT == 6
            int64_t e = ((int64_t)(d % p->x) * p->bs + slot) * p->x + d / p->x; /* planted: packing transposed */
#else
            int64_t e = ((int64_t)(d / p->x) * p->bs + slot) * p->x + d % p->x;
#endif
            K[t * p->D + d] = p->key_u8 ? e4m3(p->key_u8[kbase + e]) * p->k_scale
                                        : (double)p->key_cache[kbase + e];
        }
        for (int d = 0; d < p->Dv; ++d) {
#if ORACLE_MUTANT == 10
            int64_t e = slot * (int64_t)p->Dv + d; /* planted: V read token-major */
#else
            int64_t e = (int64_t)d * p->bs + slot;
#endif
#if ORACLE_MUTANT == 19
            V[t * p->Dv + d] = p->value_u8 ? e4m3(p->value_u8[vbase + e]) * p->k_scale /* planted: k_scale on V */
                                           : (double)p->value_cache[vbase + e];
#else
            V[t * p->Dv + d] = p->value_u8 ? e4m3(p->value_u8[vbase + e]) * p->v_scale
                                           : (double)p->value_cache[vbase + e];
#endif
        }
    }
}

/* Scaled logits z_t = scale * q . k_t for t in [t0, t1) ([PAv2] docstring
 * step 3: "scores = q @ k.T * scale"). */
static void logits(const orc_problem* p, int s, int h, const double* K, int64_t t0, int64_t t1,
                   double* z)
{
    const float* q = p->query + (int64_t)s * p->q_s + (int64_t)h * p->q_h;
    const int64_t L = p->seq_lens[s];
    for (int64_t t = t0; t < t1; ++t) {
        double acc = 0.0;
        for (int d = 0; d < p->D; ++d) acc += (double)q[d] * K[t * p->D + d];
        z[t - t0] = p->scale * acc;
#if ORACLE_MUTANT == 20
        if (p->alibi) z[t - t0] += (double)p->alibi[h] * (double)((L - 1) - t); /* planted: bias sign */
#else
        if (p->alibi) z[t - t0] += (double)p->alibi[h] * (double)(t - (L - 1)); /* R13 */
#endif
    }
}

/* Softmax-weighted average of V rows over [t0, t1): returns the max logit
 * and the sum of exp(z - max), and writes sum_t exp(z_t - max) v_t / sum
 * into o[Dv]. */
static void softmax_average(const orc_problem* p, const double* z, const double* V, int64_t t0,
                            int64_t t1, double* m_out, double* l_out, double* o)
{
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) m = fmax(m, z[t - t0]);
    double l = 0.0;
    for (int d = 0; d < p->Dv; ++d) o[d] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        double w = exp(z[t - t0] - m);
        l += w;
        for (int d = 0; d < p->Dv; ++d) o[d] += w * V[t * p->Dv + d];
    }
#if ORACLE_MUTANT == 7
    (void)l; /* planted: output left unnormalised */
#else
    for (int d = 0; d < p->Dv; ++d) o[d] /= l;
#endif
    *m_out = m;
    *l_out = l;
}

static int check_problem(const orc_problem* p)
{
    if (!p->query || !(p->key_cache || p->key_u8) || !(p->value_cache || p->value_u8) || !p->pages ||
        !p->seq_lens)
        return 0;
    if (p->S < 0 || p->H < 1 || p->Hkv < 1 || p->H % p->Hkv || p->D < 1 || p->Dv < 1 ||
        p->bs < 1 || p->x < 1 || p->D % p->x)
        return 0;
    return 1;
}

/* Unpartitioned definition ([PAv2] docstring steps 1-4 over the whole
 * sequence): out[s, h, :] = sum_t softmax(z)_t v_t. out is [S][H][Dv]. */
static int attention_impl(double* out, const orc_problem* pp)
{
    const orc_problem p = *pp;
    const int32_t S = p.S, H = p.H, Hkv = p.Hkv, D = p.D, Dv = p.Dv;
    const int32_t* seq_lens = p.seq_lens;
    if (!out || !check_problem(&p)) return ORC_EINVAL;
    int G = H / Hkv;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pair = 0; pair < (int64_t)S * Hkv; ++pair) {
        int s = (int)(pair / Hkv), kvh = (int)(pair % Hkv);
        int64_t L = seq_lens[s];
        for (int h = 0; h < H; ++h) {
            if (kv_head_of(&p, h) != kvh) continue;
            double* o = out + ((int64_t)s * H + h) * Dv;
            for (int d = 0; d < Dv; ++d) o[d] = 0.0; /* R3 */
        }
        if (L <= 0) continue;
        double* K = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* V = (double*)malloc(sizeof(double) * (size_t)(L * Dv));
        double* z = (double*)malloc(sizeof(double) * (size_t)L);
        if (!K || !V || !z) {
            free(K); free(V); free(z);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        gather_seq(&p, s, kvh, L, K, V);
        for (int h = 0; h < H; ++h) {
            if (kv_head_of(&p, h) != kvh) continue;
            double m, l;
            logits(&p, s, h, K, 0, L, z);
            softmax_average(&p, z, V, 0, L, &m, &l, out + ((int64_t)s * H + h) * Dv);
        }
        free(K); free(V); free(z);
        (void)G;
    }
    return failed ? ORC_ENOMEM : ORC_OK;
}

/* Split length of sequence s (reading R4). */
static int64_t split_len(int64_t L, const int32_t* num_splits, int s, int32_t partition_size,
                         int32_t max_num_parts)
{
    if (!num_splits) return partition_size;
    int64_t n = num_splits[s];
    if (n < 1) n = 1;
    if (n > max_num_parts) n = max_num_parts;
    int64_t c = cdiv64(L < 1 ? 1 : L, n);
    return cdiv64(c, 64) * 64;
}

/* Phase-1 intermediates per partition ([PAv2] partition kernel: per
 * (seq, head, partition) the range [p*P, min((p+1)*P, L)), online-softmax
 * max and sum, weighted V; stores max_logits, exp_sums and tmp_output).
 * Empty partitions (start >= L) store max = -inf, sum = 0 and leave tmp
 * untouched, as the page's early exit does. Layouts: tmp [S][H][Pmax][Dv],
 * max_logits and exp_sums [S][H][Pmax]. tmp holds acc / l (reading R1). */
static int partials_impl(double* tmp, double* max_logits, double* exp_sums, const orc_problem* pp,
                         const int32_t* num_splits, int32_t partition_size, int32_t max_num_parts)
{
    const orc_problem p = *pp;
    const int32_t S = p.S, H = p.H, Hkv = p.Hkv, D = p.D, Dv = p.Dv;
    const int32_t* seq_lens = p.seq_lens;
    if (!tmp || !max_logits || !exp_sums || !check_problem(&p) || max_num_parts < 1) return ORC_EINVAL;
    if (!num_splits && partition_size < 1) return ORC_EINVAL;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pair = 0; pair < (int64_t)S * Hkv; ++pair) {
        int s = (int)(pair / Hkv), kvh = (int)(pair % Hkv);
        int64_t L = seq_lens[s];
        int64_t len = split_len(L, num_splits, s, partition_size, max_num_parts);
        double* K = NULL; double* V = NULL; double* z = NULL;
        if (L > 0) {
            K = (double*)malloc(sizeof(double) * (size_t)(L * D));
            V = (double*)malloc(sizeof(double) * (size_t)(L * Dv));
            z = (double*)malloc(sizeof(double) * (size_t)L);
            if (!K || !V || !z) {
                free(K); free(V); free(z);
#pragma omp atomic write
                failed = 1;
                continue;
            }
            gather_seq(&p, s, kvh, L, K, V);
        }
        for (int h = 0; h < H; ++h) {
            if (kv_head_of(&p, h) != kvh) continue;
            int64_t base = ((int64_t)s * H + h) * max_num_parts;
            for (int64_t part = 0; part < max_num_parts; ++part) {
                int64_t t0 = part * len;
#if ORACLE_MUTANT == 9
                int64_t t1 = min64(t0 + len - 1, L); /* planted: partition drops its last token */
#else
                int64_t t1 = min64(t0 + len, L);
#endif
                if (t0 >= t1) {
                    max_logits[base + part] = -INFINITY;
                    exp_sums[base + part] = 0.0;
                    continue;
                }
                logits(&p, s, h, K, t0, t1, z);
                softmax_average(&p, z, V, t0, t1, &max_logits[base + part], &exp_sums[base + part],
                                tmp + (base + part) * Dv);
            }
        }
        free(K); free(V); free(z);
    }
    return failed ? ORC_ENOMEM : ORC_OK;
}

/* ------------------------------------------------------------------------
 * Entry points: the plain problem, and the variants of R13 / R14 (optional
 * ALiBi slopes; fp8 caches as uint8 codes with the float-cache strides).
 * ------------------------------------------------------------------------ */
#define ORC_PROBLEM_ARGS                                                             \
    const float *query, int64_t q_s, int64_t q_h, const float *key_cache, int64_t k_b, \
        int64_t k_h, const float *value_cache, int64_t v_b, int64_t v_h,              \
        const int32_t *pages, int64_t pg_s, int64_t pg_b, const int32_t *indptr,      \
        const int32_t *seq_lens, int32_t S, int32_t H, int32_t Hkv, int32_t D,        \
        int32_t Dv, int32_t bs, int32_t x, double scale
#define ORC_PROBLEM_INIT(alibi, ku8, vu8, ks, vs)                                                \
    {query, q_s, q_h, key_cache, k_b, k_h, value_cache, v_b, v_h, pages, pg_s, pg_b, indptr,    \
     seq_lens, S, H, Hkv, D, Dv, bs, x, scale, alibi, ku8, vu8, ks, vs}

int orc_attention(double* out, ORC_PROBLEM_ARGS)
{
    const orc_problem p = ORC_PROBLEM_INIT(NULL, NULL, NULL, 1.0, 1.0);
    return attention_impl(out, &p);
}
int orc_attention_v(double* out, ORC_PROBLEM_ARGS, const float* alibi, const uint8_t* key_u8,
                    const uint8_t* value_u8, double k_scale, double v_scale)
{
    const orc_problem p = ORC_PROBLEM_INIT(alibi, key_u8, value_u8, k_scale, v_scale);
    return attention_impl(out, &p);
}
int orc_partials(double* tmp, double* max_logits, double* exp_sums, ORC_PROBLEM_ARGS,
                 const int32_t* num_splits, int32_t partition_size, int32_t max_num_parts)
{
    const orc_problem p = ORC_PROBLEM_INIT(NULL, NULL, NULL, 1.0, 1.0);
    return partials_impl(tmp, max_logits, exp_sums, &p, num_splits, partition_size, max_num_parts);
}
int orc_partials_v(double* tmp, double* max_logits, double* exp_sums, ORC_PROBLEM_ARGS,
                   const int32_t* num_splits, int32_t partition_size, int32_t max_num_parts,
                   const float* alibi, const uint8_t* key_u8, const uint8_t* value_u8,
                   double k_scale, double v_scale)
{
    const orc_problem p = ORC_PROBLEM_INIT(alibi, key_u8, value_u8, k_scale, v_scale);
    return partials_impl(tmp, max_logits, exp_sums, &p, num_splits, partition_size, max_num_parts);
}

/* Phase 2 ([PAv2] _paged_attn_v2_reduce_kernel): over the n nonempty
 * partitions of the sequence, global max M = max_p m_p; rescaled sums
 * w_p = exp(m_p - M) * l_p; weights w_p / sum_p w_p; output = sum_p weight_p
 * * tmp_p. Unlike the page's MAX_NUM_PARTS cap of 1024, every partition is
 * merged. Layouts as orc_partials; out is [S][H][Dv]. */
int orc_reduce(double* out, const double* tmp, const double* max_logits, const double* exp_sums,
               const int32_t* seq_lens, const int32_t* num_splits, int32_t partition_size,
               int32_t S, int32_t H, int32_t Dv, int32_t max_num_parts)
{
    if (!out || !tmp || !max_logits || !exp_sums || !seq_lens || S < 0 || H < 1 || Dv < 1 ||
        max_num_parts < 1 || (!num_splits && partition_size < 1))
        return ORC_EINVAL;
    for (int s = 0; s < S; ++s) {
        int64_t L = seq_lens[s];
        int64_t len = split_len(L, num_splits, s, partition_size, max_num_parts);
        int64_t n = L > 0 ? min64(cdiv64(L, len), max_num_parts) : 0;
        for (int h = 0; h < H; ++h) {
            int64_t base = ((int64_t)s * H + h) * max_num_parts;
            double* o = out + ((int64_t)s * H + h) * Dv;
            for (int d = 0; d < Dv; ++d) o[d] = 0.0;
            if (n == 0) continue;
            double M = -INFINITY;
            for (int64_t q = 0; q < n; ++q) M = fmax(M, max_logits[base + q]);
            double total = 0.0;
            for (int64_t q = 0; q < n; ++q) {
#if ORACLE_MUTANT == 8
                total += exp(max_logits[base + q] - M); /* planted: sums not used */
#else
                total += exp(max_logits[base + q] - M) * exp_sums[base + q];
#endif
            }
            for (int64_t q = 0; q < n; ++q) {
#if ORACLE_MUTANT == 8
                double w = exp(max_logits[base + q] - M) / total;
#else
                double w = exp(max_logits[base + q] - M) * exp_sums[base + q] / total;
#endif
                for (int d = 0; d < Dv; ++d) o[d] += w * tmp[(base + q) * Dv + d];
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Decode metadata, [SGMETA] normal_decode_set_metadata, its docstring's steps
 * in order:
 *   1. cache_seqlens[b] = int32(seq_lens[b] + delta)
 *   2. cu_seqlens_k = exclusive prefix sum of cache_seqlens, total at [B]
 *   3. slot = req_to_token[req_pool_indices[b], col * page_size] for
 *      0 <= col < max_seq_pages (the 2-D gather; every page_size-th token
 *      slot of the request's row is the first slot of one page)
 *   4. page_table[b, col] = floor(slot / page_size)
 *   5. optional: swa_page_table[b, col] = floor(full_to_swa[slot] / page_size)
 * All arrays are addressed through element strides. page_size must be a
 * power of two (the page asserts it).
 * ------------------------------------------------------------------------ */
static int64_t floor_div64(int64_t a, int64_t b)
{
    int64_t q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

int orc_decode_metadata(int32_t* cache_seqlens, int64_t cs_stride,
                        int32_t* cu_seqlens_k, int64_t cu_stride,
                        int32_t* page_table, int64_t pt_s0, int64_t pt_s1,
                        int32_t* swa_page_table, int64_t swa_s0, int64_t swa_s1,
                        const int64_t* seq_lens, int64_t sl_stride,
                        const int32_t* req_to_token, int64_t rt_s0, int64_t rt_s1,
                        const int64_t* req_pool_indices, int64_t rpi_stride,
                        const int32_t* full_to_swa, int64_t f2s_stride,
                        int32_t batch, int32_t max_seq_pages, int32_t page_size,
                        int64_t seq_len_delta)
{
    if (batch < 0 || max_seq_pages < 0 || page_size <= 0 || (page_size & (page_size - 1)))
        return ORC_EINVAL;
    if (!cu_seqlens_k || (batch > 0 && (!cache_seqlens || !seq_lens))) return ORC_EINVAL;
    if (batch > 0 && max_seq_pages > 0 && (!page_table || !req_to_token || !req_pool_indices))
        return ORC_EINVAL;
    const int use_swa = swa_page_table != NULL && full_to_swa != NULL;

    /* steps 1 and 2 (R7: int32 wrap, done through uint32) */
    uint32_t total = 0;
    for (int32_t b = 0; b < batch; ++b) {
#if ORACLE_MUTANT == 12
        uint32_t v = (uint32_t)(uint64_t)seq_lens[(int64_t)b * sl_stride]; /* planted: delta dropped */
#else
        uint32_t v = (uint32_t)(uint64_t)(seq_lens[(int64_t)b * sl_stride] + seq_len_delta);
#endif
        cache_seqlens[(int64_t)b * cs_stride] = (int32_t)v;
#if ORACLE_MUTANT == 11
        total += v; /* planted: inclusive prefix sum */
        cu_seqlens_k[(int64_t)b * cu_stride] = (int32_t)total;
#else
        cu_seqlens_k[(int64_t)b * cu_stride] = (int32_t)total;
        total += v;
#endif
    }
    cu_seqlens_k[(int64_t)batch * cu_stride] = (int32_t)total;

    /* steps 3 to 5 */
    for (int32_t b = 0; b < batch; ++b) {
#if ORACLE_MUTANT == 15
        int64_t row = b; /* planted: pool index ignored */
#else
        int64_t row = req_pool_indices[(int64_t)b * rpi_stride];
#endif
        for (int32_t col = 0; col < max_seq_pages; ++col) {
#if ORACLE_MUTANT == 13
            int64_t tok = col; /* planted: column not scaled to a token position */
#else
            int64_t tok = (int64_t)col * page_size;
#endif
            int64_t slot = req_to_token[row * rt_s0 + tok * rt_s1];
            int64_t page = floor_div64(slot, page_size);
            page_table[(int64_t)b * pt_s0 + (int64_t)col * pt_s1] = (int32_t)page;
            if (use_swa) {
#if ORACLE_MUTANT == 14
                int64_t swa_slot = full_to_swa[page * f2s_stride]; /* planted: maps the page */
#else
                int64_t swa_slot = full_to_swa[slot * f2s_stride];
#endif
                swa_page_table[(int64_t)b * swa_s0 + (int64_t)col * swa_s1] =
                    (int32_t)floor_div64(swa_slot, page_size);
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Speculative SWA page table, [SGMETA] prepare_swa_spec_page_table_triton:
 * the page table of each of the bs requests is concatenated with the
 * expanded page table of each of its R = draft_tokens draft rows. Row m of
 * the destination (0 <= m < bs * R) belongs to request m / R; with
 * la = seq_len_a[m / R] and lb = seq_len_b[m], column n < la + lb is
 *   a[m / R, n]        for n < la   (0 when n >= LEN_A)
 *   b[m, n - la]       for n >= la  (0 when n - la >= LEN_B)
 * and columns n >= la + lb are left untouched (R12 for the table widths).
 * ------------------------------------------------------------------------ */
int orc_swa_spec_page_table(int32_t* dst, int64_t d0, int64_t d1,
                            const int32_t* a, int64_t a0, int64_t a1,
                            const int32_t* b, int64_t b0, int64_t b1,
                            const int32_t* seq_len_a, const int32_t* seq_len_b,
                            int32_t bs, int32_t len_a, int32_t len_b, int32_t draft_tokens)
{
    if (bs < 0 || len_a < 0 || len_b < 0 || draft_tokens < 1) return ORC_EINVAL;
    if (bs == 0) return ORC_OK;
    if (!dst || !seq_len_a || !seq_len_b || (len_a > 0 && !a) || (len_b > 0 && !b)) return ORC_EINVAL;
    const int64_t rows = (int64_t)bs * draft_tokens;
    for (int64_t m = 0; m < rows; ++m) {
#if ORACLE_MUTANT == 16
        const int64_t ia = m; /* planted: draft row used as the request row */
#else
        const int64_t ia = m / draft_tokens;
#endif
        const int64_t la = seq_len_a[ia], lb = seq_len_b[m];
        const int64_t end = min64(la + lb, (int64_t)len_a + len_b);
        for (int64_t n = 0; n < end; ++n) {
            int32_t v;
            if (n < la) {
                v = n < len_a ? a[ia * a0 + n * a1] : 0;
            } else {
#if ORACLE_MUTANT == 17
                const int64_t j = n; /* planted: b column not shifted by la */
#else
                const int64_t j = n - la;
#endif
                v = j < len_b ? b[m * b0 + j * b1] : 0;
            }
            dst[m * d0 + n * d1] = v;
        }
    }
    return ORC_OK;
}

/* Number of planted-mistake variants this file defines (for the tests). */
int orc_num_mutants(void) { return 20; }
int orc_mutant_id(void) { return ORACLE_MUTANT; }
