// index_kernels.hip -- integer helpers of the decode step: the flat page list,
// the split-count heuristic and the token-offset test hook.
#include <limits.h>

#include "kernels.h"

namespace pa {

// ---------------------------------------------------------------------------
// Flat page list (vLLM PR 35765, _copy_page_indices_kernel in its
// stride-robust form): workgroups (request r, part y) copy request r's
// cu[r+1] - cu[r] table entries to page_indices[cu[r] ...], reading the row
// with both strides. The copy is latency-bound: 8 x 256 lanes per row with
// four loads in flight each cover 8192 entries per memory round trip (the
// 64-request, ~4600-entry page list of the MLA batch: one round; one
// 1024-lane workgroup per row took five, 5.3 us).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_page_indices(int32_t* __restrict__ out,
                                                      const int32_t* __restrict__ bt, int64_t s0,
                                                      int64_t s1,
                                                      const int32_t* __restrict__ cu)
{
    // kPageCopyParts workgroups per request row, 4 entries per thread per
    // round with all four loads in flight before the stores
    const int r = blockIdx.x;
    const int64_t start = cu[r];
    const int64_t n = (int64_t)cu[r + 1] - start;
    const int32_t* row = bt + (int64_t)r * s0;
    const int64_t step = (int64_t)gridDim.y * blockDim.x;
    for (int64_t i0 = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i0 < n; i0 += 4 * step) {
        int32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = i0 + k * step;
            v[k] = i < n ? row[i * s1] : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = i0 + k * step;
            if (i < n) out[start + i] = v[k];
        }
    }
}

hipError_t launch_page_indices(int32_t* out, const int32_t* bt, int64_t s0, int64_t s1,
                               const int32_t* cu, int num_reqs, hipStream_t st)
{
    constexpr int kPageCopyParts = 8;
    hipLaunchKernelGGL(k_page_indices, dim3(num_reqs, kPageCopyParts), dim3(256), 0, st, out, bt, s0, s1, cu);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-count heuristic (sglang metadata.py, get_num_kv_splits_triton), one
// workgroup: block-wide max/min of the lengths, then each lane evaluates the
// formula for its sequences. The float steps follow the page's fp32
// arithmetic: fp32(max)/64, log2 (the double log2 rounded to fp32), one
// fp32 multiply by the core count, truncation to int32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
// cdiv for 1 <= a, b < 2^31 (a + b - 1 < 2^32): 32-bit unsigned division
__device__ __forceinline__ uint32_t cdiv_u32(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// 256 threads; a thread keeps the lengths it loads (kSplitHold per thread,
// all batches up to 1024 sequences) for the second pass instead of reading
// them again.
constexpr int kSplitThreads = 256, kSplitHold = 4;

__global__ __launch_bounds__(kSplitThreads) void k_num_kv_splits(int32_t* __restrict__ out,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 int num_seq, int num_group, int num_head,
                                                                 int num_kv_head, int max_kv_splits,
                                                                 int cores)
{
    __shared__ int s_max[kSplitThreads / kWave], s_min[kSplitThreads / kWave];
    const int tid = threadIdx.x;
    int held[kSplitHold];  // lengths of sequences tid + kSplitThreads * j, clamped to >= 1
    int mx = 1, mn = INT_MAX;
#pragma unroll
    for (int j = 0; j < kSplitHold; ++j) {
        const int i = tid + kSplitThreads * j;
        int L = i < num_seq ? seq_lens[i] : 1;
        L = L < 1 ? 1 : L;
        held[j] = L;
        if (i < num_seq) {
            mx = L > mx ? L : mx;
            mn = L < mn ? L : mn;
        }
    }
    for (int i = tid + kSplitThreads * kSplitHold; i < num_seq; i += kSplitThreads) {
        int L = seq_lens[i];
        L = L < 1 ? 1 : L;
        mx = L > mx ? L : mx;
        mn = L < mn ? L : mn;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        int a = __shfl_xor(mx, o, kWave), b = __shfl_xor(mn, o, kWave);
        mx = a > mx ? a : mx;
        mn = b < mn ? b : mn;
    }
    const int wave = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
        s_max[wave] = mx;
        s_min[wave] = mn;
    }
    __syncthreads();
    int64_t max_len = s_max[0], min_len = s_min[0];
#pragma unroll
    for (int w = 1; w < kSplitThreads / kWave; ++w) {
        max_len = s_max[w] > max_len ? s_max[w] : max_len;
        min_len = s_min[w] < min_len ? s_min[w] : min_len;
    }
    if (max_len * 8 < min_len * 10) min_len = max_len;
    int64_t splits1 = cdiv_u32((uint32_t)max_len, (uint32_t)min_len);
    splits1 = splits1 < max_kv_splits ? splits1 : max_kv_splits;
    const uint32_t chunk1 = cdiv_u32((uint32_t)max_len, (uint32_t)splits1);

    const float ext = (float)max_len / 64.0f;
    const float lg = (float)log2((double)ext);
    const float prod = __fmul_rn((float)cores, fmaxf(lg, 1.0f));
    const int64_t cores_ext = (int32_t)prod;

    const int64_t group = num_head / num_kv_head;
    int64_t grid;
    if (group == 1) {
        grid = (int64_t)num_seq * num_group * num_head;
    } else {
        const int64_t bh = group < 16 ? group : 16;
        grid = (int64_t)num_seq * num_group * cdiv(num_head, bh);
    }
    int64_t splits2 = cdiv(cores_ext, grid);
    splits2 = splits2 < max_kv_splits ? splits2 : max_kv_splits;
    const uint32_t chunk2 = cdiv_u32((uint32_t)max_len, (uint32_t)splits2);

    auto put = [&](int i, uint32_t L) {
        const uint32_t a = cdiv_u32(L, chunk1), b = cdiv_u32(L, chunk2);
        const int32_t n = (int32_t)(a > b ? a : b);
        for (int g = 0; g < num_group; ++g) out[(int64_t)i * num_group + g] = n;
    };
#pragma unroll
    for (int j = 0; j < kSplitHold; ++j) {
        const int i = tid + kSplitThreads * j;
        if (i < num_seq) put(i, (uint32_t)held[j]);
    }
    for (int i = tid + kSplitThreads * kSplitHold; i < num_seq; i += kSplitThreads) {
        const int L = seq_lens[i];
        put(i, (uint32_t)(L < 1 ? 1 : L));
    }
}

hipError_t launch_num_kv_splits(int32_t* out, const int32_t* seq_lens, int num_seq, int num_group,
                                int num_head, int num_kv_head, int max_kv_splits, int cores,
                                hipStream_t st)
{
    hipLaunchKernelGGL(k_num_kv_splits, dim3(1), dim3(kSplitThreads), 0, st, out, seq_lens, num_seq,
                       num_group, num_head, num_kv_head, max_kv_splits, cores);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token offsets through page_of / slot_of, the functions every decode
// kernel uses to find a token's block and slot.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_token_offsets(int64_t* __restrict__ out, int64_t out_ss,
                                                       PageList pl,
                                                       const int32_t* __restrict__ seq_lens,
                                                       int max_seq_len, int bs_shift,
                                                       int64_t block_stride, int64_t slot_stride)
{
    const int s = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t L = seq_lens[s];
    L = L < max_seq_len ? L : max_seq_len;
    if (t >= L) return;
    const int32_t* row = page_row(pl, s);
    out[(int64_t)s * out_ss + t] = token_offset(row, pl.stride_b, t, bs_shift, block_stride, slot_stride);
}

hipError_t launch_token_offsets(int64_t* out, int64_t out_ss, const PageList& pl,
                                const int32_t* seq_lens, int num_seqs, int max_seq_len,
                                int bs_shift, int64_t block_stride, int64_t slot_stride,
                                hipStream_t st)
{
    dim3 grid((max_seq_len + 255) / 256, num_seqs);
    hipLaunchKernelGGL(k_token_offsets, grid, dim3(256), 0, st, out, out_ss, pl, seq_lens,
                       max_seq_len, bs_shift, block_stride, slot_stride);
    return hipGetLastError();
}

}  // namespace pa
