// reduce.hip -- phase 2 of split-KV decode: log-sum-exp merge of the split
// outputs (paged_attention_v2_triton.py, _paged_attn_v2_reduce_kernel:
// global max, rescale by exp(m_p - M) * l_p, normalise, weighted sum).
//
// C = Dv/EPT threads cover a Dv-wide row, EPT consecutive columns each (4
// for fp32 rows, 8 for 16-bit rows: one 16-byte load either way), and NG
// thread groups take every NG-th split of one (query row, head); a
// 256-thread workgroup holds 256 / (C * NG) heads of one query row. With fixed
// partitions NG is the smallest power of two that leaves every group at
// most 4 splits, as far as the workgroup's 256 threads allow (then up to 8,
// still one round); with split counts or balanced splits, whose
// sequences mostly have a few splits, NG is the least that fills a wave.
// Each thread folds its splits into a local (max, sum, row) state, RB
// splits at a time with all their loads in flight (16-bit rows: each
// split's 16 bytes kept packed until the fold, 4 registers and not 8
// widened values, which lets 7 instead of 6 waves share a SIMD), and the groups' states
// are merged once through LDS with the same rule (M = max m_g, weights
// exp(m_g - M)): one memory round trip and one barrier. With fixed
// partitions the first batch is requested together with the sequence's
// length (slots past the split count are inside the workspaces; what they
// hold is dropped by a select, never multiplied). Otherwise only splits
// below the count are read; with balanced splits the first batch is
// requested with the length as well (every slot lies in the workspaces and
// the balanced rule fills a prefix of them). Skewed batch 13.3 -> 7.2 us
// and MLA batch 25.0 -> 17.2 us against one workgroup per head, 8 splits
// per batch and groups sized by max_num_parts.
#include <type_traits>

#include "kernels.h"

namespace pa {

constexpr int kRedMaxThreads = 256;
constexpr int kRedBatch = 8;  // splits per thread per round of loads (at most)

// RB: splits per thread per round of loads. Eight when fixed partitions give
// every group that many (one round); four with split counts or balanced
// splits, whose sequences mostly have a few splits: the smaller batch needs
// fewer registers, so more waves are resident and fewer rounds of the
// two dependent loads run one after another.
// A workgroup takes HPW = 256 / (C * NG) heads of one query row (up to 256
// threads), so the row's length and split count are loaded once for all of
// them and small per-head thread counts do not turn into many tiny
// workgroups (split counts: 8192 one-wave workgroups on the skewed batch).
template <int C, int NG> constexpr int red_heads() { return kRedMaxThreads / (C * NG) > 0 ? kRedMaxThreads / (C * NG) : 1; }

// columns per thread for split rows of element type TmpE
template <class TmpE> constexpr int red_ept() { return TmpE::size == 4 ? 4 : 8; }

// The 16 bytes of EPT consecutive partial values at p (16-byte aligned):
// four fp32 values, or eight 16-bit values kept packed as loaded (a batch
// of rows then takes 4 registers a split, not 8) and widened at the fold.
template <int EPT> using RowPiece = typename std::conditional<EPT == 4, f32x4, u32x4>::type;
template <class TmpE, int EPT>
__device__ __forceinline__ RowPiece<EPT> load_cols(const typename TmpE::storage* p)
{
    if constexpr (EPT == 4) return load_tmp4<TmpE>(p);
    else return *reinterpret_cast<const u32x4*>(p);
}
// value i of such a piece, widened
template <class TmpE, int EPT>
__device__ __forceinline__ float col_of(const RowPiece<EPT>& w, int i)
{
    if constexpr (EPT == 4) {
        return w[i];
    } else {
        using S = typename TmpE::storage;
        return to_f32(__builtin_bit_cast(S, (uint16_t)(w[i >> 1] >> (16 * (i & 1)))));
    }
}

template <class OutE, class TmpE, int DV, int NG, int RB>
__global__ __launch_bounds__(kRedMaxThreads) void k_reduce(ReduceParams p)  // C * NG * HPW = 256
{
    constexpr int EPT = red_ept<TmpE>();  // columns per thread
    constexpr int C = DV / EPT;           // threads per row
    constexpr int HPW = red_heads<C, NG>();
    __shared__ float acc_lds[HPW][NG][EPT][C];
    __shared__ float m_lds[HPW][NG], w_lds[HPW][NG];

    const int hs = threadIdx.x / (C * NG), tid = threadIdx.x % (C * NG);
    const int col = tid % C, grp = tid / C;
    // row = s * num_group + j: query token j of sequence s; heads
    // HPW*hb .. HPW*hb + HPW - 1 (past the last head: a repeat of it, not
    // stored)
    const int hblocks = (p.num_heads + HPW - 1) / HPW;
    const int row = blockIdx.x / hblocks, hraw = (blockIdx.x % hblocks) * HPW + hs;
    const bool head_ok = hraw < p.num_heads;
    const int h = head_ok ? hraw : p.num_heads - 1;
    const int s = row / p.num_group;
    const int64_t obase = (int64_t)row * p.out_ss + (int64_t)h * p.out_sh + EPT * col;

    const float* ml = p.max_logits + (int64_t)row * p.ml_ss + (int64_t)h * p.ml_sh;
    const float* es = p.exp_sums + (int64_t)row * p.ml_ss + (int64_t)h * p.ml_sh;
    using TT = typename TmpE::storage;
    const TT* tmp = reinterpret_cast<const TT*>(p.tmp) + (int64_t)row * p.tmp_ss + (int64_t)h * p.tmp_sh + EPT * col;

    const int L = p.seq_lens[s];
    // balanced splits (partition_size 0): every slot, empty ones skipped below
    const bool balanced = !p.num_splits && p.partition_size == 0;

    // this thread's splits grp, grp + NG, ...: local max M (base e), sum W
    // of exp(m_p - M) l_p, and acc = sum of exp(m_p - M) l_p tmp_p
    float M = -INFINITY, W = 0.0f;
    float acc[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc[i] = 0.0f;
    RowPiece<EPT> rows[RB];  // 16-byte pieces as loaded
    float mv[RB], lv[RB];
    auto zero_row = [&](int r) { rows[r] = RowPiece<EPT>{}; };
    // Fold one batch: an empty split (m = -inf) adds nothing; its row may
    // never have been written, so it is dropped by a select, not a multiply.
    auto fold = [&]() {
        float mb = M;
#pragma unroll
        for (int r = 0; r < RB; ++r) mb = fmaxf(mb, mv[r]);
        // mb = -inf: nothing live yet (acc, W are 0); avoids exp2(-inf + inf)
        const float f = mb == -INFINITY ? 1.0f : fast_exp2((M - mb) * kLog2e);
#pragma unroll
        for (int i = 0; i < EPT; ++i) acc[i] *= f;
        W *= f;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const bool live = mv[r] != -INFINITY;
            const float w = live ? fast_exp2((mv[r] - mb) * kLog2e) * lv[r] : 0.0f;
#pragma unroll
            for (int i = 0; i < EPT; ++i) acc[i] += live ? w * col_of<TmpE, EPT>(rows[r], i) : 0.0f;
            W += w;
        }
        M = mb;
    };

    int64_t q0 = grp;  // first split of the next batch
    // Fixed partitions: the first batch is requested before the length is
    // known, so its loads overlap the length's (long-context batch 5.8 ->
    // 5.2 us). Slots below max_num_parts lie inside the workspaces; those at
    // or past the split count are dropped once it is known (their rows and
    // statistics are never used). With split counts most of such a batch
    // would be empty slots, read for nothing (skewed batch 8.6 -> 9.4 us).
    // Balanced splits fill a prefix of the slots, most sequences more than a
    // batch of them: the first batch is requested the same way.
    const bool early = !p.num_splits;
    // Balanced splits: the statistics of the second batch and of the slot
    // after it come with the first batch, so a group with at most 2*RB
    // splits needs two dependent round trips (statistics and first rows,
    // then the second rows) instead of four, and knows where its splits end
    // without reading a batch of empty slots.
    float mv2[RB], lv2[RB], mnext = -INFINITY;
    if (early) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t q = q0 + (int64_t)r * NG;
            if (q < p.max_num_parts) {
                rows[r] = load_cols<TmpE, EPT>(tmp + q * p.tmp_sp);
                mv[r] = ml[q];
                lv[r] = es[q];
            } else {
                zero_row(r);
                mv[r] = -INFINITY;
                lv[r] = 0.0f;
            }
        }
        if (balanced) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t q = q0 + (int64_t)(RB + r) * NG;
                mv2[r] = q < p.max_num_parts ? ml[q] : -INFINITY;
                lv2[r] = q < p.max_num_parts ? es[q] : 0.0f;
            }
            const int64_t q = q0 + (int64_t)2 * RB * NG;
            mnext = q < p.max_num_parts ? ml[q] : -INFINITY;
        }
    }
    // the split count is read alongside the length (not behind a test of
    // it), and the split rule is evaluated while the first batch is in flight
    const int64_t len = balanced ? 1 : split_length(L, p.num_splits, row, p.partition_size, p.max_num_parts);
    int64_t n = 0;
    if (L > 0) {
        if (balanced) {
            n = p.max_num_parts;
        } else {
            n = ((int64_t)L + len - 1) / len;
            n = n < p.max_num_parts ? n : p.max_num_parts;
        }
    }
    if (n == 0) {  // the same for the whole workgroup (one row)
        if (grp == 0 && head_ok)
#pragma unroll
            for (int i = 0; i < EPT; ++i) store_out<OutE>(p.out, obase + i, 0.0f);
        return;
    }
    if (early) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (q0 + (int64_t)r * NG >= n) {
                mv[r] = -INFINITY;
                lv[r] = 0.0f;
            }
        }
        if (balanced) {
            // once this group meets an empty slot, every later one is empty
            bool ended = false;
#pragma unroll
            for (int r = 0; r < RB; ++r) ended |= mv[r] == -INFINITY;
            if (ended) n = q0 + 1;
        }
        fold();
        q0 += (int64_t)NG * RB;
        if (balanced && q0 < n) {  // the second batch, its statistics in hand
            bool ended = false;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                mv[r] = mv2[r];
                lv[r] = lv2[r];
                ended |= mv[r] == -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                if (mv[r] != -INFINITY)
                    rows[r] = load_cols<TmpE, EPT>(tmp + (q0 + (int64_t)r * NG) * p.tmp_sp);
                else
                    zero_row(r);
            }
            fold();
            // an empty slot in this batch or right after it ends the group
            n = ended || mnext == -INFINITY ? q0 : n;
            q0 += (int64_t)NG * RB;
        }
    }
    for (; q0 < n; q0 += (int64_t)NG * RB) {
        if (!balanced) {  // every split below n is live: all loads at once
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t q = q0 + (int64_t)r * NG;
                if (q < n) {
                    rows[r] = load_cols<TmpE, EPT>(tmp + q * p.tmp_sp);
                    mv[r] = ml[q];
                    lv[r] = es[q];
                } else {
                    zero_row(r);
                    mv[r] = -INFINITY;
                    lv[r] = 0.0f;
                }
            }
        } else {  // most slots are empty: statistics first, rows of live slots only
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t q = q0 + (int64_t)r * NG;
                mv[r] = q < n ? ml[q] : -INFINITY;
                lv[r] = q < n ? es[q] : 0.0f;
            }
            // the balanced rule fills a prefix of the slots: once this group
            // meets an empty one, every later slot is empty too
            bool ended = false;
#pragma unroll
            for (int r = 0; r < RB; ++r) ended |= mv[r] == -INFINITY;
            if (ended) n = q0 + 1;  // this batch is the group's last
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t q = q0 + (int64_t)r * NG;
                if (mv[r] != -INFINITY)
                    rows[r] = load_cols<TmpE, EPT>(tmp + q * p.tmp_sp);
                else
                    zero_row(r);
            }
        }
        fold();
    }

#pragma unroll
    for (int i = 0; i < EPT; ++i) acc_lds[hs][grp][i][col] = acc[i];
    if (col == 0) {
        m_lds[hs][grp] = M;
        w_lds[hs][grp] = W;
    }
    __syncthreads();
    if (grp != 0 || !head_ok) return;
    float Mt = m_lds[hs][0];
#pragma unroll
    for (int g = 1; g < NG; ++g) Mt = fmaxf(Mt, m_lds[hs][g]);
    float a[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) a[i] = 0.0f;
    float Wt = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float f = m_lds[hs][g] == -INFINITY ? 0.0f : fast_exp2((m_lds[hs][g] - Mt) * kLog2e);
#pragma unroll
        for (int i = 0; i < EPT; ++i) a[i] += f * acc_lds[hs][g][i][col];
        Wt += f * w_lds[hs][g];
    }
    const float inv = Wt > 0.0f ? 1.0f / Wt : 0.0f;  // no live split: zero row
#pragma unroll
    for (int i = 0; i < EPT; ++i) store_out<OutE>(p.out, obase + i, a[i] * inv);
}

bool reduce_supported(int Dv) { return Dv == 64 || Dv == 128 || Dv == 256 || Dv == 512; }

// Split groups for up to max_parts splits: cdiv(max_parts, 4) rounded up
// to a power of two, within [max(1, 64 / C), 256 / C] (C threads per row):
// as many threads as a workgroup holds, each with a batch of 4 to 8 splits
// (long-context batch with 16-bit rows, 64 splits: 8 groups of 8 -> 16
// groups of 4, phase 2 10.3 -> 8.9 us).
static int reduce_groups(int C, int max_parts)
{
    const int lo = C >= 64 ? 1 : 64 / C, hi = kRedMaxThreads / C;
    const int want = (max_parts + 3) / 4;
    int ng = lo;
    while (ng < want && ng < hi) ng *= 2;
    return ng;
}

template <class OutE, class TmpE, int DV, int NG>
static void launch_reduce_ng(const ReduceParams& p, hipStream_t st)
{
    constexpr int C = DV / red_ept<TmpE>();
    constexpr int HPW = red_heads<C, NG>();
    const int64_t hblocks = (p.num_heads + HPW - 1) / HPW;
    const dim3 grid((unsigned)((int64_t)p.num_seqs * p.num_group * hblocks)), block(C * NG * HPW);
    const bool few = p.num_splits || p.partition_size == 0 || (p.max_num_parts + NG - 1) / NG <= 4;
    if (few) hipLaunchKernelGGL((k_reduce<OutE, TmpE, DV, NG, 4>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_reduce<OutE, TmpE, DV, NG, kRedBatch>), grid, block, 0, st, p);
}

template <class OutE, class TmpE, int DV>
static void launch_reduce_dv(const ReduceParams& p, hipStream_t st)
{
    constexpr int C = DV / red_ept<TmpE>(), LO = C >= 64 ? 1 : 64 / C, HI = kRedMaxThreads / C;
    // split counts and balanced splits: one wave's worth of groups (most
    // sequences have a few splits; smaller workgroups keep every one resident)
    const bool few = p.num_splits || p.partition_size == 0;
    const int ng = few ? LO : reduce_groups(C, p.max_num_parts);
    if (ng <= LO) launch_reduce_ng<OutE, TmpE, DV, LO>(p, st);
    else if (ng <= 2 * LO || 2 * LO > HI) launch_reduce_ng<OutE, TmpE, DV, (2 * LO <= HI ? 2 * LO : HI)>(p, st);
    else launch_reduce_ng<OutE, TmpE, DV, HI>(p, st);
}

template <class OutE, class TmpE>
static hipError_t launch_reduce_t(const ReduceParams& p, int Dv, hipStream_t st)
{
    switch (Dv) {
    case 64: launch_reduce_dv<OutE, TmpE, 64>(p, st); break;
    case 128: launch_reduce_dv<OutE, TmpE, 128>(p, st); break;
    case 256: launch_reduce_dv<OutE, TmpE, 256>(p, st); break;
    case 512: launch_reduce_dv<OutE, TmpE, 512>(p, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class OutE>
static hipError_t launch_reduce_o(const ReduceParams& p, int Dv, hipStream_t st)
{
    switch (p.tmp_dtype) {
    case PA_F32: return launch_reduce_t<OutE, F32>(p, Dv, st);
    case PA_F16: return launch_reduce_t<OutE, F16>(p, Dv, st);
    case PA_BF16: return launch_reduce_t<OutE, BF16>(p, Dv, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const ReduceParams& p, int out_dtype, int Dv, hipStream_t st)
{
    switch (out_dtype) {
    case PA_F32: return launch_reduce_o<F32>(p, Dv, st);
    case PA_F16: return launch_reduce_o<F16>(p, Dv, st);
    case PA_BF16: return launch_reduce_o<BF16>(p, Dv, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
