// kernels.h -- kernel parameter blocks and host launchers inside libpagedattn.
// Validation happens in api.hip before any launcher is called; launchers
// assume valid arguments and return the hipError_t of their launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace pa {

// Phase-1 parameters (validated copy of pa_decode_args).
struct DecodeParams {
    void* tmp;         // split outputs, element type tmp_dtype (strides in elements)
    int tmp_dtype;     // PA_F32, PA_F16 or PA_BF16
    int64_t tmp_ss, tmp_sh, tmp_sp;
    float* exp_sums;
    float* max_logits;
    int64_t ml_ss, ml_sh;
    const void* q;
    int64_t q_ss, q_sh;
    const void* kc;
    int64_t k_sb, k_sh;
    const void* vc;
    int64_t v_sb, v_sh;
    PageList pl;
    const int32_t* seq_lens;
    const int32_t* num_splits;
    float scale_log2;  // scale * log2(e): logits are kept in base 2
    int num_heads, num_kv_heads, group;
    int bs_shift;
    int partition_size, max_num_parts;
    int num_seqs;
    int num_workers;  // > 0: balanced splits (grid z = workers), see pagedattn.h
    const float* alibi;  // optional ALiBi slopes [num_heads] (natural units)
    float v_scale;       // fp8 caches: value scale (1 otherwise); k_scale is in scale_log2
    bool kv_fp8;         // caches hold FP8 E4M3 codes
    int num_group;       // query tokens per sequence (rows s * num_group + j)
    int split_run;       // grouped-head matrix-core kernel: consecutive splits per workgroup
    int grid_parts;      // splits covered by the grid (set by the launcher)
};

struct ReduceParams {
    void* out;
    int64_t out_ss, out_sh;
    const void* tmp;   // element type tmp_dtype
    int tmp_dtype;
    int64_t tmp_ss, tmp_sh, tmp_sp;
    const float* exp_sums;
    const float* max_logits;
    int64_t ml_ss, ml_sh;
    const int32_t* seq_lens;
    const int32_t* num_splits;
    int num_seqs, num_heads, partition_size, max_num_parts;
    int num_group;  // query tokens per sequence: rows s * num_group + j
};

// Decode-metadata parameters (validated copy of pa_metadata_args).
struct MetadataParams {
    int32_t* cache_seqlens;
    int64_t cache_seqlens_stride;
    int32_t* cu_seqlens_k;
    int64_t cu_seqlens_k_stride;
    int32_t* page_table;
    int64_t page_table_stride0, page_table_stride1;
    int32_t* swa_page_table;  // NULL: no SWA table
    int64_t swa_page_table_stride0, swa_page_table_stride1;
    const int64_t* seq_lens;
    int64_t seq_lens_stride;
    const int32_t* req_to_token;
    int64_t req_to_token_stride0, req_to_token_stride1;
    const int64_t* req_pool_indices;
    int64_t req_pool_indices_stride;
    const int32_t* full_to_swa;
    int64_t full_to_swa_stride;
    int64_t seq_len_delta;
    int batch, max_seq_pages, shift, col_blocks;
};

// Speculative SWA page-table parameters.
struct SpecTableParams {
    int32_t* dst;
    int64_t dst_stride0, dst_stride1;
    const int32_t* a;
    int64_t a_stride0, a_stride1;
    const int32_t* b;
    int64_t b_stride0, b_stride1;
    const int32_t* seq_len_a;
    const int32_t* seq_len_b;
    int bs, len_a, len_b, draft_tokens, col_blocks;
};

// Read-stream probe parameters (validated copy of pa_read_probe's).
struct ProbeParams {
    const char* base0;
    const char* base1;  // optional
    const int32_t* pages;
    int64_t num_pages;
    int64_t page_stride, run_stride;  // bytes
    int runs_per_page;
    int pieces;  // 16-byte pieces per run
    uint32_t* sink;
};
hipError_t launch_read_probe(const ProbeParams& p, int workgroups, hipStream_t st);

// Message returned by pa_last_error() on this thread.
void set_last_error(const char* msg);

// Which phase-1 kernel family serves a problem.
enum class DecodeKernel { VALU, MFMA };

// Launchers. `parts` is the grid's split dimension.
hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int D, int Dv, int num_seqs,
                              int parts, hipStream_t st);
hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int D, int Dv, int num_seqs,
                              int parts, hipStream_t st);
bool decode_valu_supported(int dtype, int D, int Dv);
bool decode_mfma_supported(int dtype, int D, int Dv, int group, int block_size);
hipError_t launch_decode_mla(const DecodeParams& p, int dtype, int num_seqs, int parts, hipStream_t st);
bool decode_mla_supported(int dtype, int D, int Dv, int group, int block_size);

hipError_t launch_reduce(const ReduceParams& p, int out_dtype, int Dv, hipStream_t st);
bool reduce_supported(int Dv);

hipError_t launch_decode_metadata(MetadataParams p, hipStream_t st);
int64_t metadata_grid(int batch, int max_seq_pages);  // workgroups of one launch

hipError_t launch_swa_spec_page_table(SpecTableParams p, hipStream_t st);
int64_t spec_table_grid(int64_t rows, int len_a, int len_b);

hipError_t launch_page_indices(int32_t* out, const int32_t* bt, int64_t s0, int64_t s1,
                               const int32_t* cu, int num_reqs, hipStream_t st);
hipError_t launch_num_kv_splits(int32_t* out, const int32_t* seq_lens, int num_seq, int num_group,
                                int num_head, int num_kv_head, int max_kv_splits, int cores,
                                hipStream_t st);
hipError_t launch_token_offsets(int64_t* out, int64_t out_ss, const PageList& pl,
                                const int32_t* seq_lens, int num_seqs, int max_seq_len,
                                int bs_shift, int64_t block_stride, int64_t slot_stride,
                                hipStream_t st);

}  // namespace pa
