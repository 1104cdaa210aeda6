// decode_valu.hip -- phase 1 of split-KV decode on the vector ALUs
// (paged_attention_v2_triton.py, partition kernel and module docstring:
// per (seq, head, split) load q, gather the split's K/V rows through the
// block table, scores, online softmax, weighted V, store m, l and the
// normalised split output).
//
// One 64-lane wavefront per (seq, head, split). The split is walked in
// 64-token chunks:
//   QK     lane <-> token. Each lane reads its token's key row as D/x
//          16-byte pieces (x = 16 / element size values of one token are
//          contiguous in the x-packed cache) and dots it with q from LDS.
//   softmax  wave max over the chunk, running max m and per-lane partial
//          sums in base 2 (log2(e) folded into the scale).
//   PV     lane <-> value row. With block_size * element size >= 16 a lane
//          reads 16 bytes = 16/size consecutive tokens of its row; with page
//          size 1 (latent rows) a lane owns Dv/64 consecutive values of every
//          row. The chunk's probabilities are broadcast from LDS.
// Tokens past the split end are masked: their scores are -inf and their
// values are replaced by 0 before use, so NaN padding never propagates.
//
// The cache element type KE is the query's E or FP8E4M3 (codes dequantized
// as code value * k_scale / v_scale: k_scale is folded into the score scale,
// v_scale into the final normalisation). With ALiBi slopes each score gets
// slope[h] * (t - (L - 1)) (base 2 here, like the scores).
#include "kernels.h"

namespace pa {

// STREAM: every K/V byte is read by exactly one wave (group size 1), so the
// loads carry the nontemporal hint; with grouped heads the G waves of a kv
// head share the lines through the caches and use plain loads.
//
// NW waves per workgroup share one split: wave w takes the w-th of NW equal
// runs of whole 64-token chunks, and the waves' (max, sum, accumulator)
// states are merged through LDS at the end. A wave alone streams its chunks
// one after the other, so several per split keep more loads in flight.
template <class E, class KE, int D, int DV, bool ROWV, bool STREAM, int NW>
__global__ __launch_bounds__(64 * NW) void k_decode_valu(DecodeParams p)
{
    using T = typename E::storage;
    using KT = typename KE::storage;
    constexpr int X = 16 / KE::size;      // key packing
    constexpr int DVR = DV / kWave;       // value rows (or values) per lane
    __shared__ float q_lds[D];
    __shared__ float p_all[NW][kWave];

    // grid (kv head + Hkv * (g + G * seq), split), g the head within its kv
    // head's group: workgroups are dealt to the XCDs round-robin by linear
    // id, so with the kv head fastest every XCD gets an equal share of every
    // sequence's tokens whatever the length mix, and (Hkv a multiple of 8)
    // the G heads sharing a kv head's rows run on one XCD and share them in
    // its L2; the split index last spreads each split index over all XCDs.
    const int kvh_ = blockIdx.x % p.num_kv_heads, rest = blockIdx.x / p.num_kv_heads;
    // s: query row (token j of sequence seq = s / num_group, row seq * num_group + j)
    const int s = rest / p.group, h = kvh_ * p.group + rest % p.group, part = blockIdx.y;
    const int seq = s / p.num_group;
    const int wave = NW > 1 ? (int)threadIdx.x / kWave : 0;
    const int lane = (int)threadIdx.x % kWave;
    float* p_lds = p_all[wave];
    const int L = p.seq_lens[seq];
    const int64_t len = split_length(L, p.num_splits, s, p.partition_size, p.max_num_parts);
    const int64_t start = (int64_t)part * len;
    const int64_t end = (int64_t)L < start + len ? (int64_t)L : start + len;
    float* mlp = p.max_logits + (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
    float* esp = p.exp_sums + (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
    if (start >= end) {
        if (threadIdx.x == 0) {
            *mlp = -INFINITY;
            *esp = 0.0f;
        }
        return;
    }
    const int kvh = h / p.group;
    const int bs_shift = p.bs_shift;
    const int64_t bs = int64_t(1) << bs_shift;
    // Value rows of a block longer than one 16-byte piece are read piece by
    // piece; their lines must stay in L2 for the next piece, so only rows of
    // one piece take the streaming hint (with it, 16-bit rows of 16 tokens
    // were fetched 1.29x).
    const bool vstream = STREAM && bs * KE::size <= 16;

    const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)s * p.q_ss + (int64_t)h * p.q_sh;
    for (int i = threadIdx.x; i < D; i += kWave * NW) q_lds[i] = to_f32(q[i]);
    __syncthreads();
    // this wave's run: [wstart, wend), whole chunks from the split start
    const int64_t sub = NW > 1 ? ((end - start + NW - 1) / NW + kWave - 1) / kWave * kWave : end - start;
    const int64_t wstart = start + wave * sub;
    const int64_t wend = end < wstart + sub ? end : wstart + sub;

    const int32_t* row = page_row(p.pl, seq);
    const int64_t sb = p.pl.stride_b;
    const KT* kc = reinterpret_cast<const KT*>(p.kc) + (int64_t)kvh * p.k_sh;
    const KT* vc = reinterpret_cast<const KT*>(p.vc) + (int64_t)kvh * p.v_sh;
    const float slope = p.alibi ? p.alibi[h] * kLog2e : 0.0f;

    float m = -INFINITY;  // running max (base 2)
    float l = 0.0f;       // per-lane partial sum
    float acc[DVR];
#pragma unroll
    for (int r = 0; r < DVR; ++r) acc[r] = 0.0f;

    for (int64_t c0 = wstart; c0 < wend; c0 += kWave) {
        const int n = (int)((wend - c0) < kWave ? (wend - c0) : kWave);
        // ---- scores: lane <-> token (clamped to a valid token for the load)
        const int64_t t = c0 + (lane < n ? lane : n - 1);
        const KT* kp = kc + page_of(row, sb, t, bs_shift) * p.k_sb + slot_of(t, bs_shift) * X;
        float dot = 0.0f;
#pragma unroll 8
        for (int c = 0; c < D / X; ++c) {
            const u32x4 kv = STREAM ? load16_stream(kp + (int64_t)c * bs * X) : load16(kp + (int64_t)c * bs * X);
#pragma unroll
            for (int j = 0; j < X; ++j) dot += q_lds[c * X + j] * elem16<KE>(kv, j);
        }
        const float sc = lane < n ? dot * p.scale_log2 + slope * (float)(t - (L - 1)) : -INFINITY;
        const float mn = fmaxf(m, wave_max(sc));
        const float alpha = fast_exp2(m - mn);
        const float pl = lane < n ? fast_exp2(sc - mn) : 0.0f;
        l = l * alpha + pl;
        m = mn;
        p_lds[lane] = pl;
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < DVR; ++r) acc[r] *= alpha;

        // ---- weighted values
        if constexpr (!ROWV) {
            // lane <-> row dv = lane + 64*r; VT consecutive tokens per load
            constexpr int VT = X;
            if (bs >= VT) {
                // Groups of VT tokens in pairs, both pieces requested back to
                // back (a row of 16 tokens of a 16-bit cache is two pieces of
                // one line). A missing second group repeats the first one's
                // address and is not used.
                const int nv = (n + VT - 1) / VT;
                for (int v = 0; v < nv; v += 2) {
                    const bool two = v + 1 < nv;
                    const int64_t tv0 = c0 + v * VT, tv1 = two ? tv0 + VT : tv0;
                    const KT* vp0 = vc + page_of(row, sb, tv0, bs_shift) * p.v_sb + slot_of(tv0, bs_shift);
                    const KT* vp1 = vc + page_of(row, sb, tv1, bs_shift) * p.v_sb + slot_of(tv1, bs_shift);
                    u32x4 va[DVR], vb[DVR];
#pragma unroll
                    for (int r = 0; r < DVR; ++r) {
                        const int64_t ro = (int64_t)(lane + kWave * r) * bs;
                        va[r] = vstream ? load16_stream(vp0 + ro) : load16(vp0 + ro);
                        vb[r] = vstream ? load16_stream(vp1 + ro) : load16(vp1 + ro);
                    }
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        if (half == 1 && !two) break;
                        const int vv_ = v + half;
                        float pv[VT];
#pragma unroll
                        for (int j = 0; j < VT; ++j) pv[j] = p_lds[vv_ * VT + j];
                        const bool full = (vv_ + 1) * VT <= n;
#pragma unroll
                        for (int r = 0; r < DVR; ++r) {
                            const u32x4 vv = half ? vb[r] : va[r];
#pragma unroll
                            for (int j = 0; j < VT; ++j) {
                                float x = elem16<KE>(vv, j);
                                if (!full) x = (vv_ * VT + j < n) ? x : 0.0f;
                                acc[r] += pv[j] * x;
                            }
                        }
                    }
                }
            } else {
                // small blocks: one token at a time, one element per row
                for (int j = 0; j < n; ++j) {
                    const int64_t tj = c0 + j;
                    const KT* vp = vc + page_of(row, sb, tj, bs_shift) * p.v_sb + slot_of(tj, bs_shift);
                    const float pj = p_lds[j];
#pragma unroll
                    for (int r = 0; r < DVR; ++r) acc[r] += pj * to_f32(vp[(int64_t)(lane + kWave * r) * bs]);
                }
            }
        } else {
            // page size 1: lane <-> values [lane*DVR, lane*DVR + DVR) of each row
            for (int j = 0; j < n; ++j) {
                const int64_t tj = c0 + j;
                const KT* vp = vc + (int64_t)page_of(row, sb, tj, 0) * p.v_sb + lane * DVR;
                const float pj = p_lds[j];
                if constexpr (DVR * KE::size == 16) {
                    const u32x4 vv = STREAM ? load16_stream(vp) : load16(vp);
#pragma unroll
                    for (int r = 0; r < DVR; ++r) acc[r] += pj * elem16<KE>(vv, r);
                } else {
#pragma unroll
                    for (int r = 0; r < DVR; ++r) acc[r] += pj * to_f32(vp[r]);
                }
            }
        }
        wave_lds_sync();
    }

    float lsum = wave_sum(l);
    if constexpr (NW > 1) {
        // merge: M = max_w m_w, l = sum_w exp2(m_w - M) l_w, acc likewise; a
        // wave without tokens has m = -inf and weight 0 (wave 0 always has some)
        __shared__ float m_w[NW], l_w[NW];
        __shared__ float acc_w[NW][DV];
        if (lane == 0) {
            m_w[wave] = m;
            l_w[wave] = lsum;
        }
#pragma unroll
        for (int r = 0; r < DVR; ++r) acc_w[wave][ROWV ? lane * DVR + r : lane + kWave * r] = acc[r];
        __syncthreads();
        if (wave != 0) return;
        float M = m_w[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, m_w[w]);
        lsum = 0.0f;
#pragma unroll
        for (int r = 0; r < DVR; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = m_w[w] == -INFINITY ? 0.0f : fast_exp2(m_w[w] - M);
            lsum += f * l_w[w];
#pragma unroll
            for (int r = 0; r < DVR; ++r) acc[r] += f * acc_w[w][ROWV ? lane * DVR + r : lane + kWave * r];
        }
        m = M;
    }
    if (lane == 0) {
        *mlp = m * kLn2;
        *esp = lsum;
    }
    const float inv = p.v_scale / lsum;
    const int64_t out = (int64_t)s * p.tmp_ss + (int64_t)h * p.tmp_sh + (int64_t)part * p.tmp_sp;
#pragma unroll
    for (int r = 0; r < DVR; ++r) {
        const int dv = ROWV ? lane * DVR + r : lane + kWave * r;
        store_tmp1(p.tmp, p.tmp_dtype, out + dv, acc[r] * inv);
    }
}

bool decode_valu_supported(int dtype, int D, int Dv)
{
    (void)dtype;
    return (D == Dv && (D == 64 || D == 128 || D == 256)) || (D == 576 && Dv == 512);
}

// Waves per split. Two took the MHA batch's phase 1 from 85 to 79 us (fp8
// caches: 55 to 49 us); four gave the same as two.
#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 2
#endif

template <class E, class KE, int D, int DV, int NW>
static void launch_valu_nw(const DecodeParams& p, dim3 grid, hipStream_t st)
{
    const dim3 block(kWave * NW);
    const bool stream = p.group == 1;
    if (p.bs_shift == 0) {
        if (stream) hipLaunchKernelGGL((k_decode_valu<E, KE, D, DV, true, true, NW>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((k_decode_valu<E, KE, D, DV, true, false, NW>), grid, block, 0, st, p);
    } else {
        if (stream) hipLaunchKernelGGL((k_decode_valu<E, KE, D, DV, false, true, NW>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((k_decode_valu<E, KE, D, DV, false, false, NW>), grid, block, 0, st, p);
    }
}

template <class E, class KE, int D, int DV>
static hipError_t launch_valu_t(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    const dim3 grid(num_seqs * p.num_group * p.num_heads, parts);
    launch_valu_nw<E, KE, D, DV, PA_VALU_WAVES>(p, grid, st);
    return hipGetLastError();
}

template <class E, class KE>
static hipError_t launch_valu_e(const DecodeParams& p, int D, int Dv, int num_seqs, int parts,
                                hipStream_t st)
{
    if (D == 64 && Dv == 64) return launch_valu_t<E, KE, 64, 64>(p, num_seqs, parts, st);
    if (D == 128 && Dv == 128) return launch_valu_t<E, KE, 128, 128>(p, num_seqs, parts, st);
    if (D == 256 && Dv == 256) return launch_valu_t<E, KE, 256, 256>(p, num_seqs, parts, st);
    if (D == 576 && Dv == 512) return launch_valu_t<E, KE, 576, 512>(p, num_seqs, parts, st);
    return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_valu_kv(const DecodeParams& p, int D, int Dv, int num_seqs, int parts,
                                 hipStream_t st)
{
    return p.kv_fp8 ? launch_valu_e<E, FP8E4M3>(p, D, Dv, num_seqs, parts, st)
                    : launch_valu_e<E, E>(p, D, Dv, num_seqs, parts, st);
}

hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int D, int Dv, int num_seqs,
                              int parts, hipStream_t st)
{
    switch (dtype) {
    case PA_F32: return launch_valu_kv<F32>(p, D, Dv, num_seqs, parts, st);
    case PA_F16: return launch_valu_kv<F16>(p, D, Dv, num_seqs, parts, st);
    case PA_BF16: return launch_valu_kv<BF16>(p, D, Dv, num_seqs, parts, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
