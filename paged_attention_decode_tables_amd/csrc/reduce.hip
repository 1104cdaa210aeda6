// reduce.hip -- phase 2 of split-KV decode: log-sum-exp merge of the split
// outputs (paged_attention_v2_triton.py, _paged_attn_v2_reduce_kernel:
// global max, rescale by exp(m_p - M) * l_p, normalise, weighted sum).
//
// One wavefront per (seq, head); four per workgroup. Lane l owns the VPL
// consecutive output values [l*VPL, (l+1)*VPL), so each split row of
// tmp_output is read as one contiguous 4*Dv-byte run. The split weights are
// computed 64 at a time (lane <-> split) and broadcast with readlane.
#include "kernels.h"

namespace pa {

template <int VPL>
struct RowVec {
    float v[VPL];
};

template <int VPL>
__device__ __forceinline__ RowVec<VPL> load_row(const float* p)
{
    RowVec<VPL> r;
    if constexpr (VPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VPL; i += 4) {
            f32x4 t = *reinterpret_cast<const f32x4*>(p + i);
            r.v[i] = t[0];
            r.v[i + 1] = t[1];
            r.v[i + 2] = t[2];
            r.v[i + 3] = t[3];
        }
    } else if constexpr (VPL == 2) {
        float2 t = *reinterpret_cast<const float2*>(p);
        r.v[0] = t.x;
        r.v[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) r.v[i] = p[i];
    }
    return r;
}

template <class OutE, int DV>
__global__ __launch_bounds__(256) void k_reduce(ReduceParams p)
{
    constexpr int VPL = DV / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (int64_t)p.num_seqs * p.num_heads) return;
    const int s = (int)(pair / p.num_heads);
    const int h = (int)(pair % p.num_heads);
    const int64_t obase = (int64_t)s * p.out_ss + (int64_t)h * p.out_sh + lane * VPL;

    const int L = p.seq_lens[s];
    int64_t n = 0;
    if (L > 0) {
        const int64_t len = split_length(L, p.num_splits, s, p.partition_size, p.max_num_parts);
        n = ((int64_t)L + len - 1) / len;
        n = n < p.max_num_parts ? n : p.max_num_parts;
    }
    if (n == 0) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) store_out<OutE>(p.out, obase + i, 0.0f);
        return;
    }
    const float* ml = p.max_logits + (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh;
    const float* es = p.exp_sums + (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh;
    const float* tmp = p.tmp + (int64_t)s * p.tmp_ss + (int64_t)h * p.tmp_sh + lane * VPL;

    // global max over the nonempty splits
    float M = -INFINITY;
    for (int64_t q = lane; q < n; q += kWave) M = fmaxf(M, ml[q]);
    M = wave_max(M);

    float acc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc[i] = 0.0f;
    float wsum = 0.0f;
    for (int64_t q0 = 0; q0 < n; q0 += kWave) {
        const int64_t q = q0 + lane;
        float w = 0.0f;
        if (q < n) w = fast_exp2((ml[q] - M) * kLog2e) * es[q];
        wsum += w;
        const int cnt = (int)((n - q0) < kWave ? (n - q0) : kWave);
        const float* row = tmp + q0 * p.tmp_sp;
        int j = 0;
        for (; j + 4 <= cnt; j += 4) {
            RowVec<VPL> r0 = load_row<VPL>(row + (int64_t)(j + 0) * p.tmp_sp);
            RowVec<VPL> r1 = load_row<VPL>(row + (int64_t)(j + 1) * p.tmp_sp);
            RowVec<VPL> r2 = load_row<VPL>(row + (int64_t)(j + 2) * p.tmp_sp);
            RowVec<VPL> r3 = load_row<VPL>(row + (int64_t)(j + 3) * p.tmp_sp);
            const float w0 = __shfl(w, j + 0, kWave), w1 = __shfl(w, j + 1, kWave);
            const float w2 = __shfl(w, j + 2, kWave), w3 = __shfl(w, j + 3, kWave);
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                acc[i] += w0 * r0.v[i] + w1 * r1.v[i] + w2 * r2.v[i] + w3 * r3.v[i];
        }
        for (; j < cnt; ++j) {
            RowVec<VPL> r0 = load_row<VPL>(row + (int64_t)j * p.tmp_sp);
            const float w0 = __shfl(w, j, kWave);
#pragma unroll
            for (int i = 0; i < VPL; ++i) acc[i] += w0 * r0.v[i];
        }
    }
    const float inv = 1.0f / wave_sum(wsum);
#pragma unroll
    for (int i = 0; i < VPL; ++i) store_out<OutE>(p.out, obase + i, acc[i] * inv);
}

bool reduce_supported(int Dv) { return Dv == 64 || Dv == 128 || Dv == 256 || Dv == 512; }

template <class OutE>
static hipError_t launch_reduce_t(const ReduceParams& p, int Dv, hipStream_t st)
{
    const int64_t pairs = (int64_t)p.num_seqs * p.num_heads;
    dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
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
