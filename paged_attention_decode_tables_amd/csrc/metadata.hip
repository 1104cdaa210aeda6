// metadata.hip -- decode metadata in one launch (sglang
// kernels/ops/attention/metadata.py, normal_decode_set_metadata and its fused
// metadata kernels): per-request lengths, their exclusive prefix sum, and the
// page table gathered from the request -> token-slot table, with the optional
// sliding-window (SWA) table; and the speculative SWA page-table concat of the
// same page (prepare_swa_spec_page_table_triton).
//
// Workgroup 0 computes the lengths and the prefix sum; every other workgroup
// gathers kMetaCols columns of one request's row. The prefix sum is a block
// scan over tiles of kMetaThreads * kMetaPer lengths (a thread folds kMetaPer
// consecutive lengths, the wave scans with shuffles, the four wave totals go
// through LDS), carried from tile to tile, so any batch size takes one pass.
// Arithmetic is int32 with two's complement wrap, done in uint32.
#include "kernels.h"

namespace pa {

constexpr int kMetaThreads = 256;
constexpr int kMetaColsPerThread = 4;
constexpr int kMetaCols = kMetaThreads * kMetaColsPerThread;  // columns per gather workgroup
constexpr int kMetaPer = 8;                                    // lengths per thread per scan tile

__device__ __forceinline__ void meta_scan(const MetadataParams& p)
{
    __shared__ uint32_t wave_tot[kMetaThreads / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    uint32_t carry = 0;  // sum of the lengths of all earlier tiles
    for (int64_t t0 = 0; t0 < p.batch; t0 += (int64_t)kMetaThreads * kMetaPer) {
        const int64_t b0 = t0 + (int64_t)tid * kMetaPer;
        uint32_t v[kMetaPer];
        uint32_t own = 0;
#pragma unroll
        for (int i = 0; i < kMetaPer; ++i) {
            const int64_t b = b0 + i;
            v[i] = 0;
            if (b < p.batch) {
                v[i] = (uint32_t)(uint64_t)(p.seq_lens[b * p.seq_lens_stride] + p.seq_len_delta);
                p.cache_seqlens[b * p.cache_seqlens_stride] = (int32_t)v[i];
            }
            own += v[i];
        }
        // inclusive scan of the thread totals within the wave
        uint32_t inc = own;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t up = __shfl_up(inc, d, kWave);
            if (lane >= d) inc += up;
        }
        if (lane == kWave - 1) wave_tot[wave] = inc;
        __syncthreads();
        uint32_t before = carry;  // this thread's first exclusive value
        uint32_t tile = 0;
#pragma unroll
        for (int w = 0; w < kMetaThreads / kWave; ++w) {
            if (w < wave) before += wave_tot[w];
            tile += wave_tot[w];
        }
        before += inc - own;
#pragma unroll
        for (int i = 0; i < kMetaPer; ++i) {
            const int64_t b = b0 + i;
            if (b < p.batch) p.cu_seqlens_k[b * p.cu_seqlens_k_stride] = (int32_t)before;
            before += v[i];
        }
        carry += tile;
        __syncthreads();  // wave_tot is rewritten by the next tile
    }
    if (tid == 0) p.cu_seqlens_k[(int64_t)p.batch * p.cu_seqlens_k_stride] = (int32_t)carry;
}

template <bool SWA>
__global__ __launch_bounds__(kMetaThreads) void k_decode_metadata(MetadataParams p)
{
    if (blockIdx.x == 0) {
        meta_scan(p);
        return;
    }
    const int64_t wg = (int64_t)blockIdx.x - 1;
    const int b = (int)(wg / p.col_blocks);
    const int cb = (int)(wg % p.col_blocks);
    const int64_t row = p.req_pool_indices[(int64_t)b * p.req_pool_indices_stride];
    const int32_t* src = p.req_to_token + row * p.req_to_token_stride0;
    int32_t slot[kMetaColsPerThread];
    // loads first (all in flight), then the stores
#pragma unroll
    for (int j = 0; j < kMetaColsPerThread; ++j) {
        const int col = cb * kMetaCols + j * kMetaThreads + (int)threadIdx.x;
        slot[j] = col < p.max_seq_pages
                      ? src[((int64_t)col << p.shift) * p.req_to_token_stride1]
                      : 0;
    }
#pragma unroll
    for (int j = 0; j < kMetaColsPerThread; ++j) {
        const int col = cb * kMetaCols + j * kMetaThreads + (int)threadIdx.x;
        if (col >= p.max_seq_pages) continue;
        // arithmetic shift: floor division by the power-of-two page size
        p.page_table[(int64_t)b * p.page_table_stride0 + (int64_t)col * p.page_table_stride1] =
            slot[j] >> p.shift;
        if constexpr (SWA) {
            const int32_t s = p.full_to_swa[(int64_t)slot[j] * p.full_to_swa_stride];
            p.swa_page_table[(int64_t)b * p.swa_page_table_stride0 +
                             (int64_t)col * p.swa_page_table_stride1] = s >> p.shift;
        }
    }
}

// Speculative SWA page table (prepare_swa_spec_page_table_triton): one
// workgroup per (destination row, kMetaCols columns). Row m belongs to
// request m / draft; its columns below la + lb take the request's page
// table, then the draft row's, with zeros past either table's width, and the
// row stops at len_a + len_b columns. Reads are masked by the table widths
// and writes by the destination width, so any length values are safe.
__global__ __launch_bounds__(kMetaThreads) void k_swa_spec_page_table(SpecTableParams p)
{
    const int64_t wg = blockIdx.x;
    const int64_t m = wg / p.col_blocks;
    const int cb = (int)(wg % p.col_blocks);
    const int64_t ia = m / p.draft_tokens;
    const int64_t la = p.seq_len_a[ia], lb = p.seq_len_b[m];
    const int64_t width = (int64_t)p.len_a + p.len_b;
    const int64_t end = la + lb < width ? la + lb : width;
    int32_t v[kMetaColsPerThread];
#pragma unroll
    for (int j = 0; j < kMetaColsPerThread; ++j) {
        const int64_t n = (int64_t)cb * kMetaCols + j * kMetaThreads + threadIdx.x;
        v[j] = 0;
        if (n < end) {
            if (n < la) {
                if (n < p.len_a) v[j] = p.a[ia * p.a_stride0 + n * p.a_stride1];
            } else if (n - la < p.len_b) {
                v[j] = p.b[m * p.b_stride0 + (n - la) * p.b_stride1];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMetaColsPerThread; ++j) {
        const int64_t n = (int64_t)cb * kMetaCols + j * kMetaThreads + threadIdx.x;
        if (n < end) p.dst[m * p.dst_stride0 + n * p.dst_stride1] = v[j];
    }
}

int64_t spec_table_grid(int64_t rows, int len_a, int len_b)
{
    return rows * ((((int64_t)len_a + len_b) + kMetaCols - 1) / kMetaCols);
}

hipError_t launch_swa_spec_page_table(SpecTableParams p, hipStream_t st)
{
    p.col_blocks = (int)((((int64_t)p.len_a + p.len_b) + kMetaCols - 1) / kMetaCols);
    const int64_t grid = spec_table_grid((int64_t)p.bs * p.draft_tokens, p.len_a, p.len_b);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(k_swa_spec_page_table, dim3((unsigned)grid), dim3(kMetaThreads), 0, st, p);
    return hipGetLastError();
}

int64_t metadata_grid(int batch, int max_seq_pages)
{
    const int64_t col_blocks = ((int64_t)max_seq_pages + kMetaCols - 1) / kMetaCols;
    return 1 + (int64_t)batch * col_blocks;
}

hipError_t launch_decode_metadata(MetadataParams p, hipStream_t st)
{
    p.col_blocks = (int)(((int64_t)p.max_seq_pages + kMetaCols - 1) / kMetaCols);
    const int64_t grid = metadata_grid(p.batch, p.max_seq_pages);
    if (p.swa_page_table)
        hipLaunchKernelGGL((k_decode_metadata<true>), dim3((unsigned)grid), dim3(kMetaThreads), 0, st, p);
    else
        hipLaunchKernelGGL((k_decode_metadata<false>), dim3((unsigned)grid), dim3(kMetaThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace pa
