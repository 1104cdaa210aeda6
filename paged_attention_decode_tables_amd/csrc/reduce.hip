// reduce.hip -- phase 2 of split-KV decode: log-sum-exp merge of the split
// outputs (paged_attention_v2_triton.py, _paged_attn_v2_reduce_kernel:
// global max, rescale by exp(m_p - M) * l_p, normalise, weighted sum).
//
// One 256-thread workgroup per (seq, head). The Dv-wide rows are read as
// float4 columns: C = Dv/4 threads cover a row and the 256/C thread groups
// take every (256/C)-th split, so all of a (seq, head)'s split rows are
// requested at once (up to 8 loads per thread in flight). The split weights
// w_p = exp(m_p - M) * l_p are formed once per split in LDS, the column sums
// of the groups are merged through LDS, and the result is scaled by
// 1 / sum_p w_p. Splits past the sequence's count are never read.
#include "kernels.h"

namespace pa {

constexpr int kRedThreads = 256;
constexpr int kRedChunk = 1024;  // splits whose weights sit in LDS at once

__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kRedThreads / kWave; ++i) r = fmaxf(r, red[i]);
    return r;
}

__device__ __forceinline__ float block_sum(float v, float* red)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kRedThreads / kWave; ++i) r += red[i];
    return r;
}

template <class OutE, int DV>
__global__ __launch_bounds__(kRedThreads) void k_reduce(ReduceParams p)
{
    constexpr int C = DV / 4;                 // threads per row (float4 columns)
    constexpr int NG = kRedThreads / C;       // split groups
    __shared__ float w_lds[kRedChunk];
    __shared__ float red[kRedThreads / kWave];
    __shared__ f32x4 part_lds[NG > 1 ? (NG - 1) * C : 1];

    const int tid = threadIdx.x;
    const int col = tid % C, grp = tid / C;
    const int s = blockIdx.x / p.num_heads, h = blockIdx.x % p.num_heads;
    const int64_t obase = (int64_t)s * p.out_ss + (int64_t)h * p.out_sh + 4 * col;

    const int L = p.seq_lens[s];
    int64_t n = 0;
    if (L > 0) {
        const int64_t len = split_length(L, p.num_splits, s, p.partition_size, p.max_num_parts);
        n = ((int64_t)L + len - 1) / len;
        n = n < p.max_num_parts ? n : p.max_num_parts;
    }
    if (n == 0) {
        if (grp == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) store_out<OutE>(p.out, obase + i, 0.0f);
        return;
    }
    const float* ml = p.max_logits + (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh;
    const float* es = p.exp_sums + (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh;
    const float* tmp = p.tmp + (int64_t)s * p.tmp_ss + (int64_t)h * p.tmp_sh + 4 * col;

    float M = -INFINITY;
    for (int64_t q = tid; q < n; q += kRedThreads) M = fmaxf(M, ml[q]);
    M = block_max(M, red);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wpart = 0.0f;
    for (int64_t q0 = 0; q0 < n; q0 += kRedChunk) {
        const int cnt = (int)((n - q0) < kRedChunk ? (n - q0) : kRedChunk);
        __syncthreads();
        for (int j = tid; j < cnt; j += kRedThreads) {
            const float w = fast_exp2((ml[q0 + j] - M) * kLog2e) * es[q0 + j];
            w_lds[j] = w;
            wpart += w;
        }
        __syncthreads();
        const float* rows = tmp + q0 * p.tmp_sp;
        int j = grp;
        for (; j + 3 * NG < cnt; j += 4 * NG) {
            const f32x4 r0 = *reinterpret_cast<const f32x4*>(rows + (int64_t)j * p.tmp_sp);
            const f32x4 r1 = *reinterpret_cast<const f32x4*>(rows + (int64_t)(j + NG) * p.tmp_sp);
            const f32x4 r2 = *reinterpret_cast<const f32x4*>(rows + (int64_t)(j + 2 * NG) * p.tmp_sp);
            const f32x4 r3 = *reinterpret_cast<const f32x4*>(rows + (int64_t)(j + 3 * NG) * p.tmp_sp);
            acc += w_lds[j] * r0 + w_lds[j + NG] * r1 + w_lds[j + 2 * NG] * r2 + w_lds[j + 3 * NG] * r3;
        }
        for (; j < cnt; j += NG) acc += w_lds[j] * *reinterpret_cast<const f32x4*>(rows + (int64_t)j * p.tmp_sp);
    }
    const float inv = 1.0f / block_sum(wpart, red);

    if constexpr (NG > 1) {
        if (grp > 0) part_lds[(grp - 1) * C + col] = acc;
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int g2 = 1; g2 < NG; ++g2) acc += part_lds[(g2 - 1) * C + col];
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out<OutE>(p.out, obase + i, acc[i] * inv);
    }
}

bool reduce_supported(int Dv) { return Dv == 64 || Dv == 128 || Dv == 256 || Dv == 512; }

template <class OutE>
static hipError_t launch_reduce_t(const ReduceParams& p, int Dv, hipStream_t st)
{
    const int64_t pairs = (int64_t)p.num_seqs * p.num_heads;
    dim3 grid((unsigned)pairs), block(kRedThreads);
    switch (Dv) {
    case 64: hipLaunchKernelGGL((k_reduce<OutE, 64>), grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((k_reduce<OutE, 128>), grid, block, 0, st, p); break;
    case 256: hipLaunchKernelGGL((k_reduce<OutE, 256>), grid, block, 0, st, p); break;
    case 512: hipLaunchKernelGGL((k_reduce<OutE, 512>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, int out_dtype, int Dv, hipStream_t st)
{
    switch (out_dtype) {
    case PA_F32: return launch_reduce_t<F32>(p, Dv, st);
    case PA_F16: return launch_reduce_t<F16>(p, Dv, st);
    case PA_BF16: return launch_reduce_t<BF16>(p, Dv, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
