// decode_mfma.hip -- phase 1 of split-KV decode for grouped query heads on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_{bf16,f16}).
//
// What is computed is the phase-1 algorithm of paged_attention_v2_triton.py
// (module docstring: per split, scores q.K^T * scale, online softmax,
// weighted V; stores m, l and the normalised split output), for all G query
// heads that share one kv head at once, so each K/V byte is read from HBM
// once per (seq, kv head) instead of G times.
//
// One 64-lane wavefront per (split, kv head, seq); lane = 16*g + r
// (g = lane >> 4, r = lane & 15). Heads sit on the 16 MFMA columns (G <= 16,
// unused columns get q = 0 and are never stored). The split is walked in
// 32-token chunks, all in registers:
//
//   QK:  S^T[t][h] = sum_d K[t][d] Q[h][d] as two 16x16x32 products per
//        32 d (tile 0 and tile 1 of the chunk). Lane (g, r) feeds A with 8
//        consecutive d of one token: in the x = 8 packed key cache those are
//        one 16-byte piece, key_cache[blk, kvh, d/8, slot, 0:8]. Row r of
//        tile 0 holds token 8*(r/4) + r%4, of tile 1 that token + 4; with the
//        16x16 accumulator layout (lane (g, r) gets rows 4g..4g+3, column r)
//        lane (g, r) then ends up with the scores of tokens 8g..8g+7 for
//        head r.
//   softmax: running max per head (max over the lane's 8 scores, then over
//        the four lanes r, r+16, r+32, r+48), probabilities in base 2,
//        rounded to the cache type; l sums the rounded values.
//   PV:  O^T[dv][h] = sum_t V[t][dv] P[t][h], one 16x16x32 product per 16
//        value rows. The B operand wants lane (g, r) to hold P[8g..8g+7][r],
//        which is exactly what the softmax left there; the A operand wants
//        V[8g..8g+7][dv = 16*mt + r], one 16-byte piece of the value cache
//        (value_cache[blk, kvh, dv, slot:slot+8]).
// Chunks that run past the split end clamp their loads to the last valid
// 8-token group (always inside an allocated block) and mask: scores -inf,
// values 0, so NaN padding in unused slots never reaches the output.
#include "kernels.h"

namespace pa {

template <class E> struct MfmaOps;
template <> struct MfmaOps<BF16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct MfmaOps<F16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <class E, int D, int DV>
__global__ __launch_bounds__(64) void k_decode_mfma(DecodeParams p)
{
    using T = typename E::storage;
    using Ops = MfmaOps<E>;
    using vec = typename Ops::vec;
    constexpr int KS = D / 32;   // QK k-steps
    constexpr int MT = DV / 16;  // PV value-row tiles

    const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int lane = threadIdx.x, g = lane >> 4, r = lane & 15;
    const int G = p.group;
    const int h = kvh * G + r;
    const bool head_ok = r < G;

    const int L = p.seq_lens[s];
    const int64_t len = split_length(L, p.num_splits, s, p.partition_size, p.max_num_parts);
    const int64_t start = (int64_t)part * len;
    const int64_t end = (int64_t)L < start + len ? (int64_t)L : start + len;
    const int64_t mloff = (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
    if (start >= end) {
        if (head_ok && g == 0) {
            p.max_logits[mloff] = -INFINITY;
            p.exp_sums[mloff] = 0.0f;
        }
        return;
    }

    // B operand of QK: lane (g, r) holds q[h][32*ks + 8g .. +8]
    vec qv[KS];
    {
        const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)s * p.q_ss + (int64_t)h * p.q_sh + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w = head_ok ? load16(q + ks * 32) : u32x4{0, 0, 0, 0};
            qv[ks] = __builtin_bit_cast(vec, w);
        }
    }

    const int bs_shift = p.bs_shift;
    const int64_t bs = int64_t(1) << bs_shift;
    const int32_t* row = page_row(p.pl, s);
    const int64_t sb = p.pl.stride_b;
    const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)kvh * p.k_sh;
    const T* vc = reinterpret_cast<const T*>(p.vc) + (int64_t)kvh * p.v_sh;
    const int64_t last_group = (end - 1) & ~int64_t(7);

    float m = -INFINITY;  // running max of head r (base 2)
    float l = 0.0f;       // this lane's share of the running sum
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t c0 = start; c0 < end; c0 += 32) {
        const bool tail = end - c0 < 32;
        // ---- addresses: K group of row r, V group of lane group g
        int64_t tk = c0 + 8 * (r >> 2);
        tk = tk <= last_group ? tk : last_group;
        int64_t tv = c0 + 8 * g;
        tv = tv <= last_group ? tv : last_group;
        const T* kp = kc + token_block(row, sb, tk, bs_shift) * p.k_sb +
                      ((tk & (bs - 1)) + (r & 3)) * 8 + (int64_t)g * bs * 8;
        const T* vp = vc + token_block(row, sb, tv, bs_shift) * p.v_sb + (int64_t)r * bs + (tv & (bs - 1));

        // ---- loads
        u32x4 k0[KS], k1[KS], vv[MT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            k0[ks] = load16(kp + (int64_t)ks * 4 * bs * 8);
            k1[ks] = load16(kp + (int64_t)ks * 4 * bs * 8 + 32);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) vv[mt] = load16(vp + (int64_t)mt * 16 * bs);

        // ---- scores
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = Ops::mma(__builtin_bit_cast(vec, k0[ks]), qv[ks], s0);
            s1 = Ops::mma(__builtin_bit_cast(vec, k1[ks]), qv[ks], s1);
        }
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = s0[i] * p.scale_log2;
            sc[4 + i] = s1[i] * p.scale_log2;
        }
        const int64_t t0 = c0 + 8 * g;  // this lane's first token
        if (tail) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sc[j] = (t0 + j < end) ? sc[j] : -INFINITY;
        }

        // ---- online softmax
        float mloc = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mloc = fmaxf(mloc, sc[j]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const float mn = fmaxf(m, mloc);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        vec pv;
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const T e = (T)fast_exp2(sc[j] - mn);
            pv[j] = e;
            psum += (float)e;
        }
        l = l * alpha + psum;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;

        // ---- weighted values
        if (tail) {
            u32x4 keep;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                keep[w] = (t0 + 2 * w < end ? 0x0000ffffu : 0u) | (t0 + 2 * w + 1 < end ? 0xffff0000u : 0u);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vv[mt] &= keep;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = Ops::mma(__builtin_bit_cast(vec, vv[mt]), pv, acc[mt]);
    }

    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (!head_ok) return;
    if (g == 0) {
        p.max_logits[mloff] = m * kLn2;
        p.exp_sums[mloff] = l;
    }
    const float inv = 1.0f / l;
    float* out = p.tmp + (int64_t)s * p.tmp_ss + (int64_t)h * p.tmp_sh + (int64_t)part * p.tmp_sp + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(out + 16 * mt) = acc[mt] * inv;
}

bool decode_mfma_supported(int dtype, int D, int Dv, int group, int block_size)
{
    return (dtype == PA_BF16 || dtype == PA_F16) && D == Dv && (D == 64 || D == 128) &&
           group >= 2 && group <= 16 && block_size >= 8;
}

template <class E, int D>
static hipError_t launch_mfma_t(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    dim3 grid(parts, p.num_kv_heads, num_seqs), block(kWave);
    hipLaunchKernelGGL((k_decode_mfma<E, D, D>), grid, block, 0, st, p);
    return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int D, int Dv, int num_seqs,
                              int parts, hipStream_t st)
{
    if (D != Dv) return hipErrorInvalidValue;
    if (dtype == PA_BF16) {
        if (D == 64) return launch_mfma_t<BF16, 64>(p, num_seqs, parts, st);
        if (D == 128) return launch_mfma_t<BF16, 128>(p, num_seqs, parts, st);
    } else if (dtype == PA_F16) {
        if (D == 64) return launch_mfma_t<F16, 64>(p, num_seqs, parts, st);
        if (D == 128) return launch_mfma_t<F16, 128>(p, num_seqs, parts, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
