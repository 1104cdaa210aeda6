// decode_mfma.hip -- phase 1 of split-KV decode for grouped query heads on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_{bf16,f16}).
//
// What is computed is the phase-1 algorithm of paged_attention_v2_triton.py
// (module docstring: per split, scores q.K^T * scale, online softmax,
// weighted V; stores m, l and the normalised split output), for all G query
// heads that share one kv head at once, so each K/V byte is read from HBM
// once per (seq, kv head) instead of G times.
//
// One workgroup per (seq, kv head, split); its waves take contiguous runs of
// the split's chunks and merge their softmax states at the end. In a wave,
// lane = 16*g + r (g = lane >> 4, r = lane & 15). Heads sit on the 16 MFMA columns (G <= 16,
// unused columns get q = 0 and are never stored). The split is walked in
// 32-token chunks, all in registers, double-buffered (the next chunk's 16 KB
// of K/V loads are in flight while the current chunk is used), with the
// split's block ids held in a register and fetched by lane shuffles:
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

// Waves per workgroup. The chunks of a split are shared out in contiguous
// runs, one run per wave, and the waves' softmax states are merged through
// LDS at the end; several short runs per split keep the tail of the grid
// short when the splits outnumber the wave slots.
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 1
#endif
constexpr int kMfmaWaves = PA_MFMA_WAVES;
// Pipeline depth: 1 = half-chunk pipeline (one 8 KB half in flight while
// the other is used), 2 = double buffering (the next 16 KB chunk in flight).
#ifndef PA_MFMA_PIPE
#define PA_MFMA_PIPE 2
#endif
// Waves per SIMD the register budget is sized for.
#ifndef PA_MFMA_OCCUPANCY
#define PA_MFMA_OCCUPANCY (PA_MFMA_PIPE == 1 ? 3 : 2)
#endif

// BS > 0 fixes the block size at compile time (every load of a chunk is then
// an immediate offset from two base addresses); BS == 0 reads it at run time.
template <class E, int D, int DV, int BS>
__global__ __launch_bounds__(64 * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(PA_MFMA_OCCUPANCY))) void k_decode_mfma(DecodeParams p)
{
    using T = typename E::storage;
    using Ops = MfmaOps<E>;
    using vec = typename Ops::vec;
    constexpr int KS = D / 32;   // QK k-steps
    constexpr int MT = DV / 16;  // PV value-row tiles
    constexpr int W = kMfmaWaves;

    // grid (kv head + Hkv * seq, split): workgroups are dealt to the XCDs
    // round-robin by linear id. With the kv head fastest, every XCD gets an
    // equal share of every sequence's tokens (Hkv a multiple of 8: exactly
    // one kv head's), whatever the length mix; the split index last keeps
    // each split index's work (split 0 is never empty, high splits often
    // are) spread over all XCDs.
    const int kvh = blockIdx.x % p.num_kv_heads, s = blockIdx.x / p.num_kv_heads, part = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const int G = p.group;
    const int h = kvh * G + r;
    const bool head_ok = r < G;

    // token positions fit in 32 bits (lengths are int32)
    const int L = p.seq_lens[s];
    const int64_t len64 = split_length(L, p.num_splits, s, p.partition_size, p.max_num_parts);
    const int64_t start64 = (int64_t)part * len64;
    if (start64 >= (int64_t)L) {
        if (wave == 0 && head_ok && g == 0) {
            const int64_t mloff = (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
            p.max_logits[mloff] = -INFINITY;
            p.exp_sums[mloff] = 0.0f;
        }
        return;
    }
    const int start = (int)start64;
    const int end = (int)((int64_t)L < start64 + len64 ? (int64_t)L : start64 + len64);
    // this wave's run of 32-token chunks: [ca, cb)
    const int nc = (end - start + 31) >> 5;
    const int ca = wave * nc / W, cb = (wave + 1) * nc / W;

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

    const int bs_shift = BS > 0 ? __builtin_ctz(BS) : p.bs_shift;
    const int bs = 1 << bs_shift;
    const int32_t* row = page_row(p.pl, s);
    const int64_t sb = p.pl.stride_b;
    const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)kvh * p.k_sh;
    const T* vc = reinterpret_cast<const T*>(p.vc) + (int64_t)kvh * p.v_sh;
    const int last_group = (end - 1) & ~7;
    // ALiBi: slope of head r in base-2 units (0 without slopes or past the group)
    const float slope = (p.alibi && head_ok) ? p.alibi[h] * kLog2e : 0.0f;

    // Block-table window held in a register: lane i has the id of block
    // blk0 + wb + i of this wave's run; the next 64 ids are fetched one window
    // ahead. Chunks never straddle a window (runs start on 32-token
    // boundaries, so a window of 64 whole blocks ends on a chunk boundary).
    const int wstart = start + 32 * ca;
    const int wend = min(end, start + 32 * cb);
    const int blk0 = wstart >> bs_shift;
    const int nblk = ca < cb ? ((wend - 1) >> bs_shift) - blk0 + 1 : 0;
    auto fetch_window = [&](int base) -> int32_t {
        const int b = base + lane;
        return b < nblk ? row[(int64_t)(blk0 + b) * sb] : 0;
    };
    int wb = 0;
    int32_t win = fetch_window(0);
    int32_t win_next = nblk > 64 ? fetch_window(64) : 0;

    auto advance_window = [&](int c0) {
        if ((c0 >> bs_shift) - blk0 >= wb + 64) {
            wb += 64;
            win = win_next;
            if (nblk > wb + 64) win_next = fetch_window(wb + 64);
        }
    };
    auto block_of = [&](int t) -> int64_t { return __shfl(win, (t >> bs_shift) - blk0 - wb, kWave); };

    // Chunk loads. tk: this lane's 8-token key group (row r of the QK
    // tiles), tv: its value group (column group g of the PV tile); both are
    // clamped to the last valid group so every load stays inside a block
    // that holds live tokens.
    struct Tile {
        u32x4 k[2 * KS];  // K of the chunk: tile 0 (tokens 8j..8j+3), tile 1 (+4)
        u32x4 v[MT];      // V of the chunk: 16 value rows per tile
    };
    auto issue_k = [&](Tile& t, int c0) {
        const int tk = min(c0 + 8 * (r >> 2), last_group);
        const T* kp = kc + block_of(tk) * p.k_sb + (((tk & (bs - 1)) + (r & 3)) * 8 + g * bs * 8);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            t.k[2 * ks] = load16_stream(kp + ks * 4 * bs * 8);
            t.k[2 * ks + 1] = load16_stream(kp + ks * 4 * bs * 8 + 32);
        }
    };
    auto issue_v = [&](Tile& t, int c0) {
        const int tv = min(c0 + 8 * g, last_group);
        const T* vp = vc + block_of(tv) * p.v_sb + (r * bs + (tv & (bs - 1)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t.v[mt] = load16_stream(vp + mt * 16 * bs);
    };

    float m = -INFINITY;  // running max of head r (base 2)
    float l = 0.0f;       // this lane's share of the running sum
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Scores and online-softmax update for the chunk at c0 (uses kt); returns
    // the probabilities as the P.V operand and leaves alpha for the rescale.
    float alpha = 1.0f;
    auto scores = [&](Tile& t, int c0) -> vec {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = Ops::mma(__builtin_bit_cast(vec, t.k[2 * ks]), qv[ks], s0);
            s1 = Ops::mma(__builtin_bit_cast(vec, t.k[2 * ks + 1]), qv[ks], s1);
        }
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = s0[i] * p.scale_log2;
            sc[4 + i] = s1[i] * p.scale_log2;
        }
        const int t0 = c0 + 8 * g;  // this lane's first token
        if (p.alibi) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sc[j] += slope * (float)(t0 + j - (L - 1));
        }
        if (end - c0 < 32) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sc[j] = (t0 + j < end) ? sc[j] : -INFINITY;
        }
        float mloc = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mloc = fmaxf(mloc, sc[j]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const float mn = fmaxf(m, mloc);
        alpha = fast_exp2(m - mn);
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
        return pv;
    };
    // Rescale and P.V for the chunk at c0 (uses vt).
    auto weigh = [&](Tile& t, int c0, vec pv) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
        if (end - c0 < 32) {
            const int t0 = c0 + 8 * g;
            u32x4 keep;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                keep[w] = (t0 + 2 * w < end ? 0x0000ffffu : 0u) | (t0 + 2 * w + 1 < end ? 0xffff0000u : 0u);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) t.v[mt] &= keep;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = Ops::mma(__builtin_bit_cast(vec, t.v[mt]), pv, acc[mt]);
    };

#if PA_MFMA_PIPE == 1
    // Software pipeline at half-chunk granularity: once the scores of chunk
    // i are formed its K registers receive chunk i+1's keys, and once its
    // P.V is done its V registers receive chunk i+1's values, so one half of
    // a chunk (8 KB) is always in flight while the other half is used. The
    // last chunk is peeled so every wait in the loop is a fixed count; the
    // scheduling fences keep the next loads from being hoisted above the
    // math that frees their registers.
    if (ca < cb) {
        Tile t;
        issue_k(t, wstart);
        issue_v(t, wstart);
        int c0 = wstart;
        for (int i = ca; i + 1 < cb; ++i, c0 += 32) {
            advance_window(c0 + 32);
            vec pv = scores(t, c0);
            __builtin_amdgcn_sched_barrier(0);
            issue_k(t, c0 + 32);
            __builtin_amdgcn_sched_barrier(0);
            weigh(t, c0, pv);
            __builtin_amdgcn_sched_barrier(0);
            issue_v(t, c0 + 32);
            __builtin_amdgcn_sched_barrier(0);
        }
        vec pv = scores(t, c0);
        weigh(t, c0, pv);
    }
#else
    // Double buffering: the whole next chunk (16 KB) is requested before the
    // current one is used. The loop is unrolled by two so the buffers have
    // fixed registers and every wait is for exactly one tile.
    if (ca < cb) {
        Tile A, B;
        issue_k(A, wstart);
        issue_v(A, wstart);
        int c0 = wstart;
        int i = ca;
        for (; i + 2 < cb; i += 2, c0 += 64) {
            advance_window(c0 + 32);
            issue_k(B, c0 + 32);
            issue_v(B, c0 + 32);
            __builtin_amdgcn_sched_barrier(0);
            weigh(A, c0, scores(A, c0));
            __builtin_amdgcn_sched_barrier(0);
            advance_window(c0 + 64);
            issue_k(A, c0 + 64);
            issue_v(A, c0 + 64);
            __builtin_amdgcn_sched_barrier(0);
            weigh(B, c0 + 32, scores(B, c0 + 32));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (i + 1 < cb) {
            advance_window(c0 + 32);
            issue_k(B, c0 + 32);
            issue_v(B, c0 + 32);
            __builtin_amdgcn_sched_barrier(0);
            weigh(A, c0, scores(A, c0));
            __builtin_amdgcn_sched_barrier(0);
            weigh(B, c0 + 32, scores(B, c0 + 32));
        } else {
            weigh(A, c0, scores(A, c0));
        }
    }
#endif
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);

    // Merge the waves' states (max, sum, accumulator of each head) in wave 0:
    // M = max_w m_w, l = sum_w exp(m_w - M) l_w, acc = sum_w exp(m_w - M) acc_w.
    // A wave without chunks holds m = -inf and contributes nothing.
    if constexpr (W > 1) {
        __shared__ f32x4 acc_lds[W > 1 ? W - 1 : 1][MT][kWave];
        __shared__ float m_lds[W > 1 ? W - 1 : 1][16], l_lds[W > 1 ? W - 1 : 1][16];
        if (wave > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc_lds[wave - 1][mt][lane] = acc[mt];
            if (g == 0) {
                m_lds[wave - 1][r] = m;
                l_lds[wave - 1][r] = l;
            }
        }
        __syncthreads();
        if (wave > 0) return;
        float M = m;
#pragma unroll
        for (int w = 0; w < W - 1; ++w) M = fmaxf(M, m_lds[w][r]);
        const float f0 = fast_exp2(m - M);
        l *= f0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] *= f0;
        for (int w = 0; w < W - 1; ++w) {
            const float f = fast_exp2(m_lds[w][r] - M);
            l += f * l_lds[w][r];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] += f * acc_lds[w][mt][lane];
        }
        m = M;
    }

    if (!head_ok) return;
    const int64_t mloff = (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
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
    dim3 grid(num_seqs * p.num_kv_heads, parts), block(kWave * kMfmaWaves);
    switch (p.bs_shift) {
    case 4: hipLaunchKernelGGL((k_decode_mfma<E, D, D, 16>), grid, block, 0, st, p); break;
    case 5: hipLaunchKernelGGL((k_decode_mfma<E, D, D, 32>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((k_decode_mfma<E, D, D, 0>), grid, block, 0, st, p); break;
    }
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
