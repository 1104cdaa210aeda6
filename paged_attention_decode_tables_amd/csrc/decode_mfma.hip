// decode_mfma.hip -- phase 1 of split-KV decode for grouped query heads on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_{bf16,f16}).
//
// What is computed is the phase-1 algorithm of paged_attention_v2_triton.py
// (module docstring: per split, scores q.K^T * scale, online softmax,
// weighted V; stores m, l and the normalised split output), for all G query
// heads that share one kv head at once, so each K/V byte is read from HBM
// once per (seq, kv head) instead of G times.
//
// Single-wave workgroups, each walking runs of consecutive splits of one
// (seq, kv head): with fixed-size splits one run of up to four per
// workgroup; with per-sequence split counts persistent workers, each taking
// an equal share of the batch's tokens as runs of whole splits. The load
// pipeline runs through a whole run, and at each split boundary the split's
// softmax state is normalised, parked in LDS and reset; after the loop the
// run's rows leave from LDS as whole 128-byte lines. Fewer,
// longer runs cut the per-workgroup start-up and drain that dominated with
// one workgroup per 512-token split. In the
// wave, lane = 16*g + r (g = lane >> 4, r = lane & 15). Heads sit on the 16 MFMA columns (G <= 16,
// unused columns get q = 0 and are never stored). The split is walked in
// 32-token chunks, loaded in 16 KB tiles of K/V (one chunk of 16-bit caches,
// two of fp8), all in registers and double-buffered (the next tile's loads
// are in flight while the current one is used), with the split's block ids
// held in a register and fetched by lane shuffles:
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
//
// FP8 E4M3 caches (x = 16) run the same products on the query's 16-bit type:
// every E4M3 value is exact in bf16 and in f16, so codes are widened in
// registers (two per conversion instruction) and nothing is rounded that the
// 16-bit path does not round. A 16-byte key piece then holds 16 d of one
// token and feeds two k-steps: lane (g, r) takes d = 64p + 16g + 0..7 for
// k-step 2p and + 8..15 for k-step 2p + 1, and q is loaded in that order. A
// value operand is 8 codes (8 tokens of one row, an 8-byte load). k_scale is
// in the score scale, v_scale is applied with the final normalisation.
#include <type_traits>

#include "kernels.h"

namespace pa {

template <class E> struct MfmaOps;
// from_fp8(lo, hi): the 8 E4M3 codes in the bytes of lo, hi (first code in
// the low byte of lo) as 8 exact values of the 16-bit type.
template <> struct MfmaOps<BF16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ vec from_fp8(uint32_t lo, uint32_t hi)
    {
        u32x4 w;
        w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
        return __builtin_bit_cast(vec, w);
    }
};
template <> struct MfmaOps<F16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ vec from_fp8(uint32_t lo, uint32_t hi)
    {
        u32x4 w;
        w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
        return __builtin_bit_cast(vec, w);
    }
};

// Splits per workgroup at most (the host picks 1..kMfmaMaxRun so that the
// grid is about one workgroup per SIMD).
constexpr int kMfmaMaxRun = 4;
// 32-token chunks per load tile with fp8 caches (1: 8 KB tiles, 2: 16 KB).
#ifndef PA_MFMA_FP8_SUB
#define PA_MFMA_FP8_SUB 2
#endif
// Waves per SIMD the register budget is sized for (grid / persistent workers).
#ifndef PA_MFMA_OCCUPANCY
#define PA_MFMA_OCCUPANCY 2
#endif
#ifndef PA_MFMA_PERSIST_OCCUPANCY
#define PA_MFMA_PERSIST_OCCUPANCY 2
#endif

// Rows of the split outputs (tmp_output). PA_PARTIAL_NT: stored with the
// nontemporal hint.
#ifndef PA_PARTIAL_NT
#define PA_PARTIAL_NT 1
#endif

// One run of nrun consecutive splits [part0, part0 + nrun) of sequence s for
// kv head kvh (the kernel body). L is the sequence length and len64 its split
// length. BS > 0 fixes the block size at compile time (every load of a chunk
// is then an immediate offset from two base addresses); BS == 0 reads it at
// run time.
template <class E, class KE, int D, int DV, int BS, bool PERSIST>
__device__ __forceinline__ void mfma_run(const DecodeParams& p, int kvh, int s, int part0, int nrun,
                                         int L, int64_t len64)
{
    using T = typename E::storage;
    using KT = typename KE::storage;
    using Ops = MfmaOps<E>;
    using vec = typename Ops::vec;
    constexpr bool F8 = KE::size == 1;  // fp8 codes, x = 16
    constexpr int KX = F8 ? 16 : 8;     // key packing x
    constexpr int KS = D / 32;   // QK k-steps
    constexpr int MT = DV / 16;  // PV value-row tiles
    // A load tile is NSUB 32-token chunks: one for 16-bit caches, two for
    // fp8 (the same 16 KB of K/V per tile either way).
    constexpr int NSUB = F8 ? PA_MFMA_FP8_SUB : 1;
    constexpr int CH = 32 * NSUB;

    // In the persistent workers' loop the lane index is re-derived through an
    // opaque zero on every run, so nothing computed from it can be hoisted
    // out of that loop (kept live across it, such values pushed the kernel
    // past 256 registers).
    int opaque = 0;
    if constexpr (PERSIST) asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
    const int lane = (int)threadIdx.x + opaque, g = lane >> 4, r = lane & 15;
    // column r of the MFMA tiles: head hh of the kv head's group, for query
    // token qg of the sequence (query groups put their tokens side by side,
    // so every K/V byte serves all of them)
    const int G = p.group;
    const int qg = r / G, hh = r - qg * G;
    const int h = kvh * G + hh;
    const bool head_ok = qg < p.num_group;
    const int qrow = s * p.num_group + qg;  // query / output row
    const int64_t mlbase = (int64_t)qrow * p.ml_ss + (int64_t)h * p.ml_sh + part0;

    // token positions fit in 32 bits (lengths are int32)
    const int64_t start64 = (int64_t)part0 * len64;
    // splits of the run that hold tokens: [0, nlive); the rest are empty
    const int nlive = start64 < (int64_t)L
                          ? (int)min((int64_t)nrun, ((int64_t)L - start64 + len64 - 1) / len64)
                          : 0;
    if (head_ok && g == 0) {
        for (int j = nlive; j < nrun; ++j) {
            p.max_logits[mlbase + j] = -INFINITY;
            p.exp_sums[mlbase + j] = 0.0f;
        }
    }
    if (nlive == 0) return;
    const int start = (int)start64;
    const int end = (int)min((int64_t)L, start64 + (int64_t)nlive * len64);
    // the run's CH-token tiles: [ca, cb)
    const int ca = 0, cb = (end - start + CH - 1) / CH;

    // B operand of QK: lane (g, r) holds q[h][32*ks + 8g .. +8] (fp8 caches:
    // q[h][64*(ks/2) + 16g + 8*(ks%2) .. +8], the order the key pieces hold)
    vec qv[KS];
    {
        const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)qrow * p.q_ss + (int64_t)h * p.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = F8 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g;
            u32x4 w = head_ok ? load16(q + d0) : u32x4{0, 0, 0, 0};
            qv[ks] = __builtin_bit_cast(vec, w);
        }
    }

    const int bs_shift = BS > 0 ? __builtin_ctz(BS) : p.bs_shift;
    const int bs = 1 << bs_shift;
    const int32_t* row = page_row(p.pl, s);
    const int64_t sb = p.pl.stride_b;
    const KT* kc = reinterpret_cast<const KT*>(p.kc) + (int64_t)kvh * p.k_sh;
    const KT* vc = reinterpret_cast<const KT*>(p.vc) + (int64_t)kvh * p.v_sh;
    const int last_group = (end - 1) & ~7;
    // ALiBi: slope of head r in base-2 units (0 without slopes or past the group)
    const float slope = (p.alibi && head_ok) ? p.alibi[h] * kLog2e : 0.0f;

    // Block-table window held in a register: lane i has the id of block
    // blk0 + wb + i of the run; the next 64 ids are fetched one window
    // ahead. Tiles never straddle a window: split starts are multiples of 64
    // tokens, so runs start on tile boundaries, and a window of 64 whole
    // blocks (block size >= 8) ends on one.
    const int wstart = start + CH * ca;
    const int wend = min(end, start + CH * cb);
    const int blk0 = wstart >> bs_shift;
    const int nblk = ca < cb ? ((wend - 1) >> bs_shift) - blk0 + 1 : 0;
    auto fetch_window = [&](int base) -> int32_t {
        const int b = base + lane;
        return b < nblk ? page_of(row, sb, (int64_t)(blk0 + b) << bs_shift, bs_shift) : 0;
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
    // Key pieces per chunk and MFMA tile: one per k-step, or (fp8) one per
    // pair of k-steps.
    constexpr int KP = F8 ? KS / 2 : KS;
    using VPiece = typename std::conditional<F8, u32x2, u32x4>::type;
    struct Tile {
        u32x4 k[NSUB][2 * KP];  // K of each chunk: MFMA tile 0 (tokens 8j..8j+3), tile 1 (+4)
        VPiece v[NSUB][MT];     // V of each chunk: 16 value rows per MFMA tile, 8 tokens each
    };
    // Chunks past the split end (the second chunk of a tail tile) load the
    // clamped group like any other masked tokens.
    auto issue_k = [&](Tile& t, int c0) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
            const int tk = min(c0 + 32 * u + 8 * (r >> 2), last_group);
            // piece (4*kp + g) of the token's D/KX pieces
            const KT* kp = kc + block_of(tk) * p.k_sb + ((slot_of(tk, bs_shift) + (r & 3)) * KX + g * bs * KX);
#pragma unroll
            for (int kp_ = 0; kp_ < KP; ++kp_) {
                t.k[u][2 * kp_] = load16_stream(kp + kp_ * 4 * bs * KX);
                t.k[u][2 * kp_ + 1] = load16_stream(kp + kp_ * 4 * bs * KX + 4 * KX);
            }
        }
    };
    auto issue_v = [&](Tile& t, int c0) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
            const int tv = min(c0 + 32 * u + 8 * g, last_group);
            const KT* vp = vc + block_of(tv) * p.v_sb + (r * bs + slot_of(tv, bs_shift));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (F8) t.v[u][mt] = load8_stream(vp + mt * 16 * bs);
                else t.v[u][mt] = load16_stream(vp + mt * 16 * bs);
            }
        }
    };

    float m = -INFINITY;  // running max of head r (base 2)
    float l = 0.0f;       // this lane's share of the running sum
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Scores and online-softmax update for the chunk at c0 (uses kt); returns
    // the probabilities as the P.V operand and leaves alpha for the rescale.
    float alpha = 1.0f;
    auto scores = [&](Tile& t, int u, int c0) -> vec {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (F8) {
#pragma unroll
            for (int kp_ = 0; kp_ < KP; ++kp_) {
                const u32x4 a = t.k[u][2 * kp_], b = t.k[u][2 * kp_ + 1];
                s0 = Ops::mma(Ops::from_fp8(a[0], a[1]), qv[2 * kp_], s0);
                s1 = Ops::mma(Ops::from_fp8(b[0], b[1]), qv[2 * kp_], s1);
                s0 = Ops::mma(Ops::from_fp8(a[2], a[3]), qv[2 * kp_ + 1], s0);
                s1 = Ops::mma(Ops::from_fp8(b[2], b[3]), qv[2 * kp_ + 1], s1);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s0 = Ops::mma(__builtin_bit_cast(vec, t.k[u][2 * ks]), qv[ks], s0);
                s1 = Ops::mma(__builtin_bit_cast(vec, t.k[u][2 * ks + 1]), qv[ks], s1);
            }
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
        mloc = across32(across16(mloc, MaxOp{}), MaxOp{});
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
    auto weigh = [&](Tile& t, int u, int c0, vec pv) {
        // Once the running maxima settle, alpha is 1 in every lane: the
        // rescale is skipped for the whole wave then (a scalar branch).
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
        }
        if (end - c0 < 32) {
            const int t0 = c0 + 8 * g;
            if constexpr (F8) {
                u32x2 keep;  // byte j of word w: token t0 + 4w + j
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    uint32_t k = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) k |= (t0 + 4 * w + j < end ? 0xffu : 0u) << (8 * j);
                    keep[w] = k;
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) t.v[u][mt] &= keep;
            } else {
                u32x4 keep;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    keep[w] = (t0 + 2 * w < end ? 0x0000ffffu : 0u) | (t0 + 2 * w + 1 < end ? 0xffff0000u : 0u);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) t.v[u][mt] &= keep;
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (F8) {
                const u32x2 v = t.v[u][mt];
                acc[mt] = Ops::mma(Ops::from_fp8(v[0], v[1]), pv, acc[mt]);
            } else {
                acc[mt] = Ops::mma(__builtin_bit_cast(vec, t.v[u][mt]), pv, acc[mt]);
            }
        }
    };
    // Split boundaries inside the run: when a tile ends one (and the run goes
    // on), the split's state is normalised into LDS slot `parked` and reset.
    // LDS traffic counts apart from the vector-memory waits of the pipeline.
    // [max(1, split_run - 1)][MT][64] rows, then [split_run - 1][32] m, l
    extern __shared__ f32x4 park[];
    float* park_ml = reinterpret_cast<float*>(park + (p.split_run > 1 ? p.split_run - 1 : 1) * MT * kWave);
    int parked = 0;
    int64_t next_boundary = start64 + len64;
    auto flush = [&](float* m_out, float* l_out, f32x4* rows) {
        const float lt = across32(across16(l, SumOp{}), SumOp{});
        const float inv = p.v_scale / lt;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) rows[mt * kWave] = acc[mt] * inv;
        if (g == 0) {
            *m_out = m * kLn2;
            *l_out = lt;
        }
    };
    // Scores, softmax and P.V of every chunk of the tile at c0.
    auto use = [&](Tile& t, int c0) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u) weigh(t, u, c0 + 32 * u, scores(t, u, c0 + 32 * u));
        if ((int64_t)(c0 + CH) >= next_boundary && c0 + CH < end) {
            flush(park_ml + 32 * parked + r, park_ml + 32 * parked + 16 + r,
                  park + parked * MT * kWave + lane);
            ++parked;
            next_boundary += len64;
            m = -INFINITY;
            l = 0.0f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // Double buffering: the whole next tile (16 KB) is requested before the
    // current one is used. The loop is unrolled by two so the buffers have
    // fixed registers and every wait is for exactly one tile.
    if (ca < cb) {
        Tile A, B;
        issue_k(A, wstart);
        issue_v(A, wstart);
        int c0 = wstart;
        int i = ca;
        for (; i + 2 < cb; i += 2, c0 += 2 * CH) {
            advance_window(c0 + CH);
            issue_k(B, c0 + CH);
            issue_v(B, c0 + CH);
            __builtin_amdgcn_sched_barrier(0);
            use(A, c0);
            __builtin_amdgcn_sched_barrier(0);
            advance_window(c0 + 2 * CH);
            issue_k(A, c0 + 2 * CH);
            issue_v(A, c0 + 2 * CH);
            __builtin_amdgcn_sched_barrier(0);
            use(B, c0 + CH);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (i + 1 < cb) {
            advance_window(c0 + CH);
            issue_k(B, c0 + CH);
            issue_v(B, c0 + CH);
            __builtin_amdgcn_sched_barrier(0);
            use(A, c0);
            __builtin_amdgcn_sched_barrier(0);
            use(B, c0 + CH);
        } else {
            use(A, c0);
        }
    }
    // The run's rows leave from LDS, read across the lanes, so that
    // consecutive lanes write consecutive 16-byte pieces of one row and every
    // store instruction covers whole 128-byte lines (from registers a store
    // covers 64 bytes of each of its 16 rows). The parked splits go first;
    // the last split then takes slot 0.
    const float lt = across32(across16(l, SumOp{}), SumOp{});
    const int cols = G * p.num_group;  // live columns
    constexpr int NCH = DV / 4;        // 16-byte pieces per row
    // Piece k of column c (values 4k .. 4k+3) in the park layout.
    auto parked_piece = [&](int slot, int c, int k) -> f32x4 {
        return park[(slot * MT + (k >> 2)) * kWave + 16 * (k & 3) + c];
    };
    auto rows_out = [&](int slot, int split) {
        auto row_at = [&](int c) -> int64_t {  // element offset of column c's row
            const int cq = c / G, ch = c - cq * G;
            return (int64_t)(s * p.num_group + cq) * p.tmp_ss + (int64_t)(kvh * G + ch) * p.tmp_sh +
                   (int64_t)split * p.tmp_sp;
        };
        if (p.tmp_dtype == PA_F32) {
            for (int e = lane; e < cols * NCH; e += kWave) {
                const int c = e / NCH, k = e - c * NCH;  // column, piece
                store_tmp4<PA_PARTIAL_NT>(p.tmp, PA_F32, row_at(c) + 4 * k, parked_piece(slot, c, k));
            }
        } else {
            // 16-bit rows: 8 values a lane, 16-byte stores like the fp32 rows
            // (measured: phase 2 reads rows written in 8-byte pieces slower)
            constexpr int NC8 = DV / 8;
            const bool bf = p.tmp_dtype == PA_BF16;
            for (int e = lane; e < cols * NC8; e += kWave) {
                const int c = e / NC8, k2 = e - c * NC8;
                const f32x4 a = parked_piece(slot, c, 2 * k2), b = parked_piece(slot, c, 2 * k2 + 1);
                const u32x4 w = bf ? u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                           pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])}
                                   : u32x4{pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]),
                                           pack_f16x2(b[0], b[1]), pack_f16x2(b[2], b[3])};
                u32x4* at = reinterpret_cast<u32x4*>(p.tmp) + ((row_at(c) + 8 * k2) >> 3);
                if constexpr (PA_PARTIAL_NT) __builtin_nontemporal_store(w, at);
                else *at = w;
            }
        }
    };
    wave_lds_sync();  // other lanes' parked rows
    for (int j = 0; j < parked; ++j) rows_out(j, part0 + j);
    wave_lds_sync();  // slot 0 read out before it is rewritten
    {
        const float inv = p.v_scale / lt;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) park[mt * kWave + lane] = acc[mt] * inv;
    }
    wave_lds_sync();
    rows_out(0, part0 + parked);
    if (!head_ok) return;
    if (g == 0) {
        p.max_logits[mlbase + parked] = m * kLn2;
        p.exp_sums[mlbase + parked] = lt;
        for (int j = 0; j < parked; ++j) {
            p.max_logits[mlbase + j] = park_ml[32 * j + r];
            p.exp_sums[mlbase + j] = park_ml[32 * j + 16 + r];
        }
    }
}

// Work units of a split for the persistent workers' balance: its tokens
// plus a fixed charge for what every split costs whatever its length
// (normalising and writing its row, a pipeline restart at run ends).
// Skewed batch, phase 1 with a charge of 0 / 64 / 128 / 256 / 512 tokens:
// bf16 caches 334 / 330 / 331 / 333 / 334 us, fp8 200 / 196 / 194 / 200 /
// 195 us.
#ifndef PA_MFMA_SPLIT_COST
#define PA_MFMA_SPLIT_COST 128
#endif

// A sequence's splits: length, live count and work units (tokens plus the
// per-split charge; lengths <= 0 have no split).
struct SeqSplits {
    int64_t len;
    int nl;
    int64_t cost;
};
__device__ __forceinline__ SeqSplits seq_splits(const DecodeParams& p, int L, int count)
{
    if (L <= 0) return SeqSplits{1, 0, 0};
    const int n = count < 1 ? 1 : (count > p.max_num_parts ? p.max_num_parts : count);
    const int64_t len = p.num_splits ? ((((int64_t)L + n - 1) / n + 63) & ~int64_t(63)) : (int64_t)p.partition_size;
    const int nl = (int)(((int64_t)L + len - 1) / len);
    return SeqSplits{len, nl, (int64_t)L + (int64_t)PA_MFMA_SPLIT_COST * nl};
}

// The split count of sequence s (1 without counts).
__device__ __forceinline__ int seq_count(const DecodeParams& p, int s)
{
    return p.num_splits ? p.num_splits[(int64_t)s * p.num_group] : 1;
}

// Work units of the whole batch, summed by one wave.
__device__ __forceinline__ int64_t batch_cost(const DecodeParams& p)
{
    const int S = p.num_seqs;
    int64_t t = 0;
    for (int b = 0; b < S; b += 4 * kWave) {
        int v[4], c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = b + j * kWave + (int)threadIdx.x;
            v[j] = s < S ? p.seq_lens[s] : 0;
            c[j] = s < S ? seq_count(p, s) : 1;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) t += seq_splits(p, v[j], c[j]).cost;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, kWave);
    return uniform_i64(t);
}

// Lane i's value, as a wave-uniform (scalar) value.
__device__ __forceinline__ int lane_value(int v, int i) { return __builtin_amdgcn_readlane(v, i); }
__device__ __forceinline__ int64_t lane_value(int64_t v, int i)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, i);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), i);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int64_t wave_scan_i64(int64_t v)
{
    const int lane = threadIdx.x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int64_t u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

// Persistent workers for per-sequence split counts. The batch's work units
// (each split's tokens plus a fixed per-split charge), in sequence and
// split order, are numbered 0..T-1. Worker u (of NU) of kv head kvh takes
// every split whose first unit falls in [u*T/NU, (u+1)*T/NU): each worker
// gets the same share of work to within one split, no workgroup is spent on
// an empty split, and a worker's consecutive splits of one sequence run
// through one load pipeline (runs of up to split_run). The splits and their
// partials are exactly those of the one-workgroup-per-split grid.
template <class E, class KE, int D, int DV, int BS>
__device__ __forceinline__ void mfma_worker(const DecodeParams& p)
{
    const int Hkv = p.num_kv_heads, S = p.num_seqs, ng = p.num_group;
    const int NU = (int)(gridDim.x / Hkv);
    const int kvh = (int)blockIdx.x % Hkv, u = (int)blockIdx.x / Hkv;
    const int lane = threadIdx.x;
    const int64_t T = batch_cost(p);
    // [X0, X1) = [floor(T*u/NU), floor(T*(u+1)/NU)) without overflow
    const int64_t tq = T / NU, tr = T % NU;
    const int64_t X0 = tq * u + tr * u / NU;
    const int64_t X1 = tq * (u + 1) + tr * (u + 1) / NU;

    // Walk the sequences 64 at a time (lane i holds sequence bj + i; the
    // lengths of four such blocks are loaded together): find the one holding
    // unit X0, then take splits until their starts reach X1. Split sp of a
    // sequence whose units start at Cs starts at Cs + sp * (len + charge).
    int64_t before = 0;  // work units of the sequences before block bj
    for (int b = 0; b < S && before < X1; b += 4 * kWave) {
        int Lq[4], nq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sl = b + j * kWave + lane;
            Lq[j] = sl < S ? p.seq_lens[sl] : 0;
            nq[j] = sl < S ? seq_count(p, sl) : 1;
        }
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
            const int bj = b + j * kWave;
            if (bj >= S || before >= X1) break;
            const int Lr = j == 0 ? Lq[0] : j == 1 ? Lq[1] : j == 2 ? Lq[2] : Lq[3];
            const int nr = j == 0 ? nq[0] : j == 1 ? nq[1] : j == 2 ? nq[2] : nq[3];
            const int64_t incl = wave_scan_i64(seq_splits(p, Lr, nr).cost);
            const int64_t blk_end = before + lane_value(incl, kWave - 1);
            if (blk_end > X0) {
                // sequences of this block that end past X0 and start before X1
                // (their splits are recomputed as scalars: fewer registers
                // live across the runs)
                for (int i = 0; i < kWave && bj + i < S; ++i) {
                    const int Ls = lane_value(Lr, i);
                    const SeqSplits sq = seq_splits(p, Ls, lane_value(nr, i));
                    const int64_t cost = sq.cost;
                    const int64_t Cs = before + lane_value(incl, i) - cost;
                    if (Cs >= X1) break;
                    if (cost == 0 || Cs + cost <= X0) continue;
                    const int64_t len = sq.len;
                    const int nl = sq.nl;
                    const int64_t unit = len + PA_MFMA_SPLIT_COST;  // units from one split start to the next
                    int sp = Cs < X0 ? (int)((X0 - Cs + unit - 1) / unit) : 0;
                    while (sp < nl) {
                        const int64_t st = Cs + sp * unit;
                        if (st >= X1) break;
                        int nrun = (int)min((int64_t)(nl - sp), (X1 - st + unit - 1) / unit);
                        nrun = min(nrun, p.split_run);
                        mfma_run<E, KE, D, DV, BS, true>(p, kvh, bj + i, sp, nrun, Ls, len);
                        sp += nrun;
                    }
                }
            }
            before = blk_end;
        }
    }

    // Splits at or past a sequence's end hold -inf / 0: worker u marks them
    // for sequences u, u + NU, ... (its kv head's columns).
    const int G = p.group, cols = G * ng;
    for (int s = u; s < S; s += NU) {
        const int Ls = p.seq_lens[s];
        int nl = 0;
        if (Ls > 0) {
            const int64_t len = split_length(Ls, p.num_splits, s * ng, p.partition_size, p.max_num_parts);
            nl = (int)(((int64_t)Ls + len - 1) / len);
        }
        const int ne = p.max_num_parts - nl;
        for (int idx = lane; idx < cols * ne; idx += kWave) {
            const int c = idx / ne, sp = nl + idx % ne;
            const int qg = c / G, hh = c - qg * G;
            const int64_t at = (int64_t)(s * ng + qg) * p.ml_ss + (int64_t)(kvh * G + hh) * p.ml_sh + sp;
            p.max_logits[at] = -INFINITY;
            p.exp_sums[at] = 0.0f;
        }
    }
}

// Phase-1 kernel. PERSIST: persistent workers (per-sequence split counts).
// Otherwise the grid is (kv head + Hkv * seq, run of splits): workgroups are
// dealt to the XCDs round-robin by linear id. With the kv head fastest, every
// XCD gets an equal share of every sequence's tokens (Hkv a multiple of 8:
// exactly one kv head's), whatever the length mix; the run index last keeps
// each run index's work (the first is never empty, late ones often are)
// spread over all XCDs. Persistent workers keep the kv head fastest too.
// Waves per SIMD: persistent workers over fp8 caches with a run-time block
// size take the whole register file (at two they spill a few registers).
template <class KE, int BS, bool PERSIST>
constexpr int mfma_occupancy()
{
    return !PERSIST ? PA_MFMA_OCCUPANCY : (BS == 0 && KE::size == 1) ? 1 : PA_MFMA_PERSIST_OCCUPANCY;
}

template <class E, class KE, int D, int DV, int BS, bool PERSIST>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(mfma_occupancy<KE, BS, PERSIST>()))) void k_decode_mfma(DecodeParams p)
{
    if constexpr (PERSIST) {
        mfma_worker<E, KE, D, DV, BS>(p);
    } else {
        const int kvh = blockIdx.x % p.num_kv_heads, s = blockIdx.x / p.num_kv_heads;
        // runs in reverse order: late runs exist only for long sequences and
        // are the longest, so they are dispatched first and the grid ends on
        // short work
        const int part0 = (int)(gridDim.y - 1 - blockIdx.y) * p.split_run;  // first split of the run
        const int nrun = min(p.split_run, p.grid_parts - part0);
        const int L = p.seq_lens[s];
        const int64_t len64 = split_length(L, p.num_splits, s * p.num_group, p.partition_size, p.max_num_parts);
        mfma_run<E, KE, D, DV, BS, false>(p, kvh, s, part0, nrun, L, len64);
    }
}

// Any 1..16 columns: with a single one (MHA, one query token) the tiles
// waste 15/16 of the matrix-core work, but the products cost the same per
// cache byte as with 16, and the load pipeline beats the vector kernel's
// (MHA batch: f16 79 vs 81 us, fp8 46 vs 50 us per step).
bool decode_mfma_supported(int dtype, int D, int Dv, int group, int block_size)
{
    return (dtype == PA_BF16 || dtype == PA_F16) && D == Dv && (D == 64 || D == 128) &&
           group >= 1 && group <= 16 && block_size >= 8;
}

// Compute units of the current device (cached per device).
static int device_cus()
{
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Splits per workgroup with fixed-size splits: enough that the grid is about
// one workgroup per SIMD (four per compute unit of the current device), at
// most kMfmaMaxRun, and at most an eighth of the split count, so a run
// never holds a large share of a sequence (with short ragged sequences,
// runs measured slower: the MHA batch, 4 splits at most, went 79 -> 83 us
// with runs of 4).
static int pick_split_run(int64_t units, int parts)
{
    int64_t run = units / (4 * (int64_t)device_cus());
    run = run < parts / 8 ? run : parts / 8;
    return (int)(run < 1 ? 1 : run > kMfmaMaxRun ? kMfmaMaxRun : run);
}

// Per-sequence split counts run on persistent workers: this many per
// compute unit (two per SIMD), each taking runs of up to PA_MFMA_WORKER_RUN
// splits (three keep eight workers' parked splits within the LDS of a
// compute unit). A worker scans the batch's lengths once, so very large
// batches keep the one-workgroup-per-split grid. Measured on the skewed
// batch (phase 1): one workgroup per split 370 us; workers 4/CU with runs
// of 4 at one wave per SIMD 329 us, at two 339 us (register-limited);
// 8/CU with runs of 3, 2, 1: 329, 333, 337 us; 16/CU with runs of 2: 342 us.
#ifndef PA_MFMA_WORKERS_PER_CU
#define PA_MFMA_WORKERS_PER_CU 8
#endif
#ifndef PA_MFMA_WORKER_RUN
#define PA_MFMA_WORKER_RUN 3
#endif
constexpr int kMfmaPersistMaxSeqs = 2048;

template <class E, class KE, int D, bool PERSIST>
static void launch_mfma_bs(const DecodeParams& p, dim3 grid, size_t lds, hipStream_t st)
{
    switch (p.bs_shift) {
    case 4: hipLaunchKernelGGL((k_decode_mfma<E, KE, D, D, 16, PERSIST>), grid, dim3(kWave), lds, st, p); break;
    case 5: hipLaunchKernelGGL((k_decode_mfma<E, KE, D, D, 32, PERSIST>), grid, dim3(kWave), lds, st, p); break;
    default: hipLaunchKernelGGL((k_decode_mfma<E, KE, D, D, 0, PERSIST>), grid, dim3(kWave), lds, st, p); break;
    }
}

template <class E, class KE, int D>
static hipError_t launch_mfma_t(DecodeParams p, int num_seqs, int parts, hipStream_t st)
{
    p.grid_parts = parts;
    const bool persist = p.num_splits && num_seqs <= kMfmaPersistMaxSeqs;
    dim3 grid;
    if (persist) {
        p.split_run = PA_MFMA_WORKER_RUN;
        const int64_t want = (int64_t)PA_MFMA_WORKERS_PER_CU * device_cus();
        const int64_t nu = (want + p.num_kv_heads - 1) / p.num_kv_heads;  // workers per kv head
        grid = dim3((unsigned)(nu * p.num_kv_heads));
    } else {
        p.split_run = p.num_splits ? 1 : pick_split_run((int64_t)num_seqs * p.num_kv_heads * parts, parts);
        grid = dim3(num_seqs * p.num_kv_heads, (parts + p.split_run - 1) / p.split_run);
    }
    if (p.split_run < 1 || p.split_run > kMfmaMaxRun) return hipErrorInvalidValue;
    // row slots (at least one: a run's last split leaves through slot 0), then m, l
    const size_t slots = p.split_run > 1 ? p.split_run - 1 : 1;
    const size_t lds = slots * (D / 16) * kWave * sizeof(f32x4) + (size_t)(p.split_run - 1) * 32 * sizeof(float);
    if (persist) launch_mfma_bs<E, KE, D, true>(p, grid, lds, st);
    else launch_mfma_bs<E, KE, D, false>(p, grid, lds, st);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_mfma_e(const DecodeParams& p, int D, int num_seqs, int parts, hipStream_t st)
{
    if (p.kv_fp8) {
        if (D == 64) return launch_mfma_t<E, FP8E4M3, 64>(p, num_seqs, parts, st);
        if (D == 128) return launch_mfma_t<E, FP8E4M3, 128>(p, num_seqs, parts, st);
    } else {
        if (D == 64) return launch_mfma_t<E, E, 64>(p, num_seqs, parts, st);
        if (D == 128) return launch_mfma_t<E, E, 128>(p, num_seqs, parts, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int D, int Dv, int num_seqs,
                              int parts, hipStream_t st)
{
    if (D != Dv) return hipErrorInvalidValue;
    if (dtype == PA_BF16) return launch_mfma_e<BF16>(p, D, num_seqs, parts, st);
    if (dtype == PA_F16) return launch_mfma_e<F16>(p, D, num_seqs, parts, st);
    return hipErrorInvalidValue;
}

}  // namespace pa
