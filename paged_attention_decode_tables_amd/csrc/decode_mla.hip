// decode_mla.hip -- phase 1 of split-KV decode for the MLA-style layout:
// many query heads (G = 64 or 128) over one latent kv head whose cache row
// holds both the key (all D = 576 values) and the value (its first Dv = 512
// values), page size 1. What is computed is the phase-1 algorithm of
// paged_attention_v2_triton.py (module docstring: per split, scores
// q.K^T * scale, online softmax, weighted V; stores m, l and the normalised
// split output); the value rows are the leading Dv columns of the key rows,
// so every latent byte is read from HBM once per split.
//
// One workgroup per (seq, kv head, split) serves all G heads with NW = G/32
// waves; wave w owns query heads 32w .. 32w+31 (lane = 32*hl + c32, head c32
// of the wave). The 32x32 matrix-core tiles make every latent byte staged in
// LDS feed 32 heads per read. The split is walked in 32-token chunks:
//
//   staging  the chunk's 32 latent rows are copied HBM -> LDS by direct
//            global-to-LDS loads (no registers hold data in flight) into a
//            ring of kMlaBuf chunk slots, kMlaBuf-1 chunks ahead. 16-byte
//            piece pc of row t sits at column pc ^ swz(t) (within groups of
//            8 pieces), swz(t) = ((t2 ^ t1) << 2) | (t1 << 1) | t3, which
//            puts the rows one operand read touches on distinct LDS banks
//            (rows two apart share a bank offset, 1152 B = 32 mod 64
//            dwords). Page ids are staged in LDS.
//   QK       S^T[t][h] = sum_d K[t][d] Q[h][d] on v_mfma_f32_32x32x16: the 32
//            tokens are the rows (A operand: 16 bytes of a latent row from
//            LDS), the wave's 32 heads the columns (B operand: q in
//            registers). A-row m reads token perm(m) = 16*(m>>4) +
//            8*((m>>2)&1) + 4*((m>>3)&1) + (m&3); with the accumulator layout
//            (lane 32*hl + c32, register r: row 8*(r>>2) + 4*hl + (r&3),
//            column c32) lane (hl, c32) then holds head c32's scores of tokens
//            16*(r>>3) + 8*hl + (r&7): tokens 8hl..8hl+7 and 16+8hl..16+8hl+7,
//            i.e. the two P.V B operands of the chunk, with no data movement.
//   softmax  running max per head over the lane's 16 scores and lane l^32;
//            probabilities rounded to the cache type.
//   PV       O^T[dv][h] = sum_t V[t][dv] P[t][h] on v_mfma_f32_32x32x16 per 32
//            value columns and 16 tokens: A = V[t0..t0+7][dv] for the lane's
//            column, two ds_read_b64_tr_b16 of the token-major rows (within
//            a 16-lane group, lane i receives value (i mod 4) of the 8-byte
//            pieces addressed by lanes i/4 + 4j, so lane a addresses row
//            t0 + a/4, columns 4(a%4) .. +3 of its 16-column half).
// Tokens past the split end are loaded from the last valid row (a real,
// finite row) and masked: scores -inf, probabilities 0.
#include <type_traits>
#include <utility>

#include "kernels.h"

namespace pa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class E> struct MlaOps;
template <> struct MlaOps<BF16> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct MlaOps<F16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and nothing else (gfx9 encoding: vmcnt bits 3:0 and 15:14).
__host__ __device__ constexpr int waitcnt_vm(int n)
{
    return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8);
}

// 16-byte direct HBM -> LDS copy: lane i's piece lands at lds_dst + 16 i.
// The builtin only exists for the device pass (in the host pass it makes
// clang drop the kernel's launch stub), hence the guard.
__device__ __forceinline__ void lds_copy16(const void* src, u32x4* lds_dst)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
#else
    (void)src;
    (void)lds_dst;
#endif
}

// LDS reads as inline assembly, with the byte offset as an immediate. The
// builtin form of the transposed read makes the compiler wait for every
// outstanding global-to-LDS copy before it, which would drain the copy ring
// on every chunk; here the ring's own vmcnt wait and barrier already order
// each read after the copies it consumes. The compiler does not track these
// reads, so a result is used only after lds_wait() has passed through it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t lds_addr)
{
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "n"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16(uint32_t lds_addr)
{
    s16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "n"(OFF));
    return v;
}

// Waits until at most N LDS operations of this wave are outstanding. LDS
// operations complete in issue order, so every read issued before the last
// N has landed; the values are threaded through the wait so nothing that
// uses them can be scheduled above it.
template <int N, class V>
__device__ __forceinline__ void lds_wait(V& v)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}
template <int N, class V>
__device__ __forceinline__ void lds_wait(V& v0, V& v1)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v0), "+v"(v1) : "n"(N));
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// max and sum of x over lanes l and l ^ 32
__device__ __forceinline__ float half_max(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float half_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Largest divisor of `ins` that is at most `nw` (waves issuing the copies).
__host__ __device__ constexpr int loader_waves(int ins, int nw)
{
    int best = 1;
    for (int d = 1; d <= nw; ++d)
        if (ins % d == 0) best = d;
    return best;
}

// LDS column offset of the pieces of ring row t (XORed into the piece index
// within each group of 8 pieces): bit 2 = t2 ^ t1, bit 1 = t1, bit 0 = t3.
// Rows t and t + 2 share LDS banks (a row is 1152 B, 32 mod 64 dwords); bit
// 2 puts their 64-byte value groups on different banks, so the transposed
// P.V reads (rows t0 .. t0 + 3 in one instruction) are conflict-free. With
// t2 alone there, they took two extra cycles each (measured). Over the 8
// rows of one parity the offsets are a permutation, so the 16-row QK reads
// stay conflict-free.
__host__ __device__ constexpr int mla_swz(int t) { return ((((t >> 2) ^ (t >> 1)) & 1) << 2) | (t & 2) | ((t >> 3) & 1); }

#ifndef PA_MLA_BUF
#define PA_MLA_BUF 4
#endif
#ifndef PA_MLA_KAHEAD
#define PA_MLA_KAHEAD 8
#endif
#ifndef PA_MLA_VAHEAD
#define PA_MLA_VAHEAD 6
#endif
constexpr int kMlaChunk = 32;             // tokens per chunk
constexpr int kMlaBuf = PA_MLA_BUF;       // chunk slots in the LDS ring
constexpr int kMlaPageWin = 1024;         // page ids staged in LDS at a time
constexpr int kMlaKAhead = PA_MLA_KAHEAD; // QK operand reads in flight ahead of their MFMAs
constexpr int kMlaVAhead = PA_MLA_VAHEAD; // PV MFMAs whose operand reads are in flight ahead
constexpr int kMlaHeadsPerWave = 32;

// Wave-wide int64 inclusive prefix sum and max of an int.
__device__ __forceinline__ int64_t wave_incl_sum_i64(int64_t v, int lane)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t up = __shfl_up(v, d, kWave);
        if (lane >= d) v += up;
    }
    return v;
}
__device__ __forceinline__ int wave_max_i32(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

// ALIBI: scores carry the slopes' bias (a separate instance, so the plain
// kernel keeps its registers).
// BAL = false: one workgroup per (seq, kv head, split) of the fixed or
// per-sequence split rule. BAL = true: balanced splits, one workgroup per
// (token range, kv head).
template <class E, int NW, bool BAL, bool ALIBI>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_decode_mla(DecodeParams p)
{
    using T = typename E::storage;
    using Ops = MlaOps<E>;
    using vec8 = typename Ops::vec8;
    constexpr int D = 576, DV = 512;
    constexpr int CT = kMlaChunk;
    constexpr int PR = D * (int)sizeof(T) / 16;  // 16-byte pieces per latent row (72)
    constexpr int RB = PR * 16;                   // bytes per latent row
    constexpr int INS = CT * PR / 64;             // copy instructions per chunk
    constexpr int LW = loader_waves(INS, NW);     // waves that issue copies
    constexpr int IPW = INS / LW;                 // copies per loader wave per chunk
    constexpr int KS = D / 16;                    // QK k-steps
    constexpr int MT = DV / 32;                   // PV value-column tiles
    constexpr int NB = kMlaBuf;
    constexpr int HPW = kMlaHeadsPerWave;
    static_assert(CT * PR % 64 == 0, "chunk must be a whole number of copy instructions");
    static_assert(PR % 8 == 0, "row pieces must be a multiple of 8 for the swizzle");
    static_assert(KS % 4 == 0 && MT % 2 == 0, "tiling");
    static_assert(IPW * (NB - 2) <= 63, "vmcnt is a 6-bit field");

    __shared__ u32x4 ring[NB][CT * PR];
    __shared__ int32_t page_lds[kMlaPageWin];
    __shared__ int rerun_flag;

    const int ngroups = p.group / (HPW * NW);
    const int hg = blockIdx.y % ngroups, kq = blockIdx.y / ngroups;
    // query token qg of every sequence (rows s * num_group + qg)
    const int qg = kq % p.num_group, kvh = kq / p.num_group;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, c32 = lane & 31, hl = lane >> 5;
    const int h0 = kvh * p.group + hg * HPW * NW;  // first head of the workgroup
    const int h = h0 + wave * HPW + c32;

    // One split (or balanced piece): tokens [start, end) of sequence s, its
    // statistics and normalised output stored in split slot `part`.
    auto piece = [&](const int s, const int part, const int start, const int end) {
    __syncthreads();  // the previous piece's LDS reads are done
    // With balanced splits the pieces run in a loop. The lane and head
    // indices are then re-derived through an opaque zero, so the compiler
    // cannot hoist what depends on them out of that loop: kept live across
    // it, they pushed the loop over chunks past the register file (spills
    // in it cost a quarter of the kernel's time).
    int opaque = 0;
    if constexpr (BAL) asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
    const int lane = (int)(threadIdx.x & 63) + opaque, c32 = lane & 31, hl = lane >> 5;
    const int wave = (int)(threadIdx.x >> 6) + opaque;
    const int h = h0 + opaque + wave * HPW + c32;
    const int nc = (end - start + CT - 1) / CT;

    // B operand of QK: lane (hl, c32) holds q[h][16*ks + 8*hl .. +8]
    vec8 qv[KS];
    {
        const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)(s * p.num_group + qg) * p.q_ss + (int64_t)h * p.q_sh + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qv[ks] = __builtin_bit_cast(vec8, load16(q + ks * 16));
    }

    const int32_t* row = page_row(p.pl, s);
    const int64_t sb = p.pl.stride_b;
    const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)kvh * p.k_sh;
    // ALiBi: head c32's slope in base-2 units (0 without slopes). Scores then
    // grow toward the end of the sequence, so a split usually passes the
    // first chunk's reference by more than the headroom and runs twice.
    const int L = ALIBI ? p.seq_lens[s] : 0;
    const float slope = ALIBI ? p.alibi[h] * kLog2e : 0.0f;

    // page ids of tokens [wbase, wbase + kMlaPageWin) of this split
    int wbase = start;
    auto stage_pages = [&](int base) {
        const int n = min(kMlaPageWin, end - base);
        for (int i = threadIdx.x; i < n; i += 64 * NW) page_lds[i] = row[(int64_t)(base + i) * sb];
    };
    stage_pages(wbase);
    __syncthreads();

    // copy chunk `c` (tokens start + CT*c ...) into ring slot c % NB
    auto issue = [&](int c) {
        if (wave >= LW) return;
        const int c0 = start + CT * c;
        u32x4* dst = &ring[c % NB][0];
        int32_t pg[IPW];  // all page ids first: one LDS round trip per chunk
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int t = ((wave * IPW + j) * 64 + lane) / PR;
            pg[j] = page_lds[min(c0 + t, end - 1) - wbase];
        }
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int ins = wave * IPW + j;
            const int piece = ins * 64 + lane;
            const int t = piece / PR, pc = piece % PR;
            const T* src = kc + (int64_t)pg[j] * p.k_sb + (int64_t)((pc ^ mla_swz(t)) * 8);
            lds_copy16(src, dst + ins * 64);
        }
    };

    // Fixed reference: probabilities are taken against mref, head c32's max
    // over the split's first chunk, and never rescaled, so the 256
    // accumulators are only ever touched by MFMAs. While no later score
    // passes mref by more than kHeadroom (base 2), p <= 2^kHeadroom and the
    // fp32 sums stay finite for value magnitudes below 2^(126 - kHeadroom -
    // log2 tokens). A split where some score does pass it is run a second
    // time with mref = the split's true max (known after the first pass), so
    // every p <= 1. The true max is kept apart and (m, l) are brought to it
    // at the end, so the stored statistics are the exact max logit and sum
    // of exp(z - max). p is rounded to the cache type before the P.V product,
    // so the headroom must keep 2^kHeadroom finite there: bf16 reaches 2^127,
    // f16 only 65504 < 2^16 (2^16 would round to +inf).
    constexpr float kHeadroom = std::is_same<E, F16>::value ? 15.0f : 64.0f;
    float mref = -INFINITY;  // reference max of head c32 (base 2)
    float mtrue = -INFINITY; // true running max of head c32 (base 2)
    float l = 0.0f;          // this lane's share of sum_t exp2(z_t - mref)
    bool over = false;       // a score of head c32 passed mref + kHeadroom
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][i] = 0.0f;

    // QK operand addresses: A-row c32 reads ring row perm(c32); piece
    // 2*ks + hl of it sits at column 8*(ks>>2) + ((2*(ks&3) + hl) ^ swz), i.e.
    // four base addresses (ks mod 4) plus 128*(ks/4) as the immediate.
    const int trow = 16 * (c32 >> 4) + 8 * ((c32 >> 2) & 1) + 4 * ((c32 >> 3) & 1) + (c32 & 3);
    const int ksw = mla_swz(trow);
    uint32_t kb_lane[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) kb_lane[q4] = trow * RB + 16 * ((2 * q4 + hl) ^ ksw);
    // PV operand addresses: read (kk, rd) of value tile mt covers rows
    // t = 16kk + 8hl + 4rd + a/4 (a = lane & 15) and value columns
    // 32mt + 16*g16 + 4*(a&3) .. +3 (g16 = (lane >> 4) & 1): piece
    // 4mt + 2*g16 + ((a&3) >> 1) at column 4*(mt ^ rd ^ t1) + low, with
    // t1 = (a >> 3) & 1 (bit 1 of the row) and low = 2*(g16 ^ (a >> 3)) +
    // (((a & 3) >> 1) ^ hl), 8 bytes in when a is odd. As the immediate
    // kk*16*RB + rd*4*RB + 64*(mt ^ rd); the lane's t1 then moves the
    // address by +64 when mt ^ rd is even and -64 when it is odd, so there
    // are two lane bases (vb_lane for even, vb_lane_odd for odd).
    uint32_t vb_lane, vb_lane_odd;
    {
        const int a = lane & 15, g16 = (lane >> 4) & 1, t1 = (a >> 3) & 1;
        const int low = 2 * (g16 ^ (a >> 3)) + (((a & 3) >> 1) ^ hl);
        const uint32_t vb = (8 * hl + (a >> 2)) * RB + 16 * low + 8 * (a & 1);
        vb_lane = vb + 64 * t1;
        vb_lane_odd = vb - 64 * t1;  // t1 = 1 only for rows >= 2: no wrap
    }

    // scores of chunk c for this lane's 16 tokens (base 2, masked past the
    // split end) and their max over both lane halves (head c32). One
    // accumulator: a second does not fit beside q and the 256 output
    // accumulators without spilling.
    auto scores = [&](int c, float (&sc)[16]) -> float {
        const int c0 = start + CT * c;
        const uint32_t bufa =
            (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)&ring[c % NB][0]);
        constexpr int RA = kMlaKAhead < KS ? kMlaKAhead : KS;
        u32x4 kr[KS];
        auto kread = [&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            kr[ks] = lds_read_b128<128 * (ks >> 2)>(bufa + kb_lane[ks & 3]);
        };
        static_for<RA>(kread);
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
        static_for<KS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int issued = (i + RA < KS) ? i + RA : KS;
            lds_wait<issued - i - 1>(kr[i]);
            sacc = Ops::mma(__builtin_bit_cast(vec8, kr[i]), qv[i], sacc);
            if constexpr (i + RA < KS) kread(std::integral_constant<int, i + RA>{});
            __builtin_amdgcn_sched_barrier(0);  // keep wait -> MFMA -> next read in order
        });
        float mloc = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = c0 + 16 * (r >> 3) + 8 * hl + (r & 7);
            float z = sacc[r] * p.scale_log2;
            if constexpr (ALIBI) z += slope * (float)(t - (L - 1));
            sc[r] = t < end ? z : -INFINITY;
            mloc = fmaxf(mloc, sc[r]);
        }
        return half_max(mloc);
    };

    // probabilities of chunk c against mref, and their weighted value rows
    auto weigh = [&](int c, const float (&sc)[16]) {
        const uint32_t slot =
            (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)&ring[c % NB][0]);
        const uint32_t vbase = slot + vb_lane, vbase_odd = slot + vb_lane_odd;
        // MFMA j (0 .. 2*MT-1) is (kk = j / MT, mt = j % MT): all tiles of the
        // first 16 tokens, then of the second, so consecutive MFMAs update
        // different accumulators
        constexpr int NJ = 2 * MT;
        constexpr int RA = kMlaVAhead < NJ ? kMlaVAhead : NJ;
        s16x4 vr[NJ][2];
        auto vread = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int kk = j / MT, mt = j % MT;
            vr[j][0] = lds_read_tr16<kk * 16 * RB + 64 * mt>((mt & 1) ? vbase_odd : vbase);
            vr[j][1] = lds_read_tr16<kk * 16 * RB + 4 * RB + 64 * (mt ^ 1)>(((mt ^ 1) & 1) ? vbase_odd : vbase);
        };
        static_for<RA>(vread);
        __builtin_amdgcn_sched_barrier(0);

        vec8 pv[2];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const T e = (T)fast_exp2(sc[r] - mref);
            pv[r >> 3][r & 7] = e;
            psum += (float)e;
        }
        l += psum;
        static_for<NJ>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int issued = (j + RA < NJ) ? j + RA : NJ;
            lds_wait<2 * (issued - j - 1)>(vr[j][0], vr[j][1]);
            const u32x4 a = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[j][0], vr[j][0], 0, 1)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[j][0], vr[j][0], 2, 3)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[j][1], vr[j][1], 0, 1)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[j][1], vr[j][1], 2, 3))};
            acc[j % MT] = Ops::mma(__builtin_bit_cast(vec8, a), pv[j / MT], acc[j % MT]);
            if constexpr (j + RA < NJ) vread(std::integral_constant<int, j + RA>{});
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Ring pipeline: chunks c+1 .. c+NB-1 are in flight while chunk c is
    // used. Copies complete in issue order, so before chunk c a loader wave
    // waits until at most IPW copies per later chunk remain outstanding
    // (all of them in the last NB-2 chunks); the barrier then makes every
    // wave's copies visible and frees the slot chunk c-1 used, which the
    // copy of chunk c+NB-1 reuses.
    // chunk c's copies are visible to every wave; chunk c+NB-1 is issued
    auto advance = [&](int c) {
        if (c + NB - 2 < nc)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(IPW * (NB - 2)));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        // A plain s_barrier: __syncthreads() would add a workgroup fence that
        // waits for every outstanding copy. The copies this barrier publishes
        // are covered by the explicit wait above; the compiler fences keep
        // LDS accesses on their side of the barrier.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const int cn = c + NB - 1;
        if (cn < nc) {
            const int tlast = min(start + CT * cn + CT, end) - 1;
            if (tlast >= wbase + kMlaPageWin) {  // next page window (all waves here)
                wbase = start + CT * cn;
                stage_pages(wbase);
                __syncthreads();
            }
            issue(cn);
        }
    };
    // one pass over the split
    auto run = [&]() {
        // q (first pass) or the previous pass's copies are complete, so no
        // wait inside the loop has to cover them
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        for (int c = 0; c < NB - 1 && c < nc; ++c) issue(c);
        for (int c = 0; c < nc; ++c) {
            float sc[16];
            advance(c);
            const float mloc = scores(c, sc);
            mtrue = fmaxf(mtrue, mloc);
            mref = mref == -INFINITY ? mloc : mref;
            over |= mloc > mref + kHeadroom;
            weigh(c, sc);
        }
    };

    if (threadIdx.x == 0) rerun_flag = 0;
    run();
    if (over) rerun_flag = 1;  // benign race: every writer stores 1
    __syncthreads();
    if (rerun_flag) {  // uniform across the workgroup
        mref = mtrue;
        l = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][i] = 0.0f;
        if (wbase != start) {
            wbase = start;
            stage_pages(wbase);
        }
        __syncthreads();  // every wave is done with the ring and the page window
        run();
    }

    l = half_sum(l);
    const int64_t mloff = (int64_t)(s * p.num_group + qg) * p.ml_ss + (int64_t)h * p.ml_sh + part;
    if (hl == 0) {
        p.max_logits[mloff] = mtrue * kLn2;
        p.exp_sums[mloff] = l * fast_exp2(mref - mtrue);
    }
    // lane (hl, c32), register 4i + j of tile mt holds value column
    // 32mt + 8i + 4hl + j of head c32
    const float inv = 1.0f / l;
    float* out = p.tmp + (int64_t)(s * p.num_group + qg) * p.tmp_ss + (int64_t)h * p.tmp_sh + (int64_t)part * p.tmp_sp + 4 * hl;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(out + 32 * mt + 8 * i) =
                f32x4{acc[mt][4 * i], acc[mt][4 * i + 1], acc[mt][4 * i + 2], acc[mt][4 * i + 3]} * inv;
    };

    if constexpr (!BAL) {
        const int s = blockIdx.x, part = blockIdx.z;
        const int L = p.seq_lens[s];
        const int64_t len64 = split_length(L, p.num_splits, s * p.num_group, p.partition_size, p.max_num_parts);
        const int64_t start64 = (int64_t)part * len64;
        if (start64 >= (int64_t)L) {  // empty split: the page's early exit
            if (hl == 0) {
                const int64_t mloff = (int64_t)(s * p.num_group + qg) * p.ml_ss + (int64_t)h * p.ml_sh + part;
                p.max_logits[mloff] = -INFINITY;
                p.exp_sums[mloff] = 0.0f;
            }
            return;
        }
        piece(s, part, (int)start64, (int)((int64_t)L < start64 + len64 ? (int64_t)L : start64 + len64));
        return;
    }

    // ---- balanced splits: worker w = blockIdx.x takes tokens [w*U, (w+1)*U)
    // of all sequences concatenated (lengths <= 0 count as 0)
    constexpr int BT = 64 * NW;
    constexpr int GH = HPW * NW;  // heads of this workgroup
    __shared__ int64_t bal_w64[NW];
    __shared__ int bal_w32[NW];
    __shared__ int64_t bal_off[BT];
    __shared__ int bal_len[BT];
    __shared__ int bal_first, bal_last;
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    // m = -inf, l = 0 in slots [k0, max_num_parts) of sequence s, all heads
    // here (all threads of the workgroup together)
    auto mark_empty = [&](int s, int k0) {
        for (int e = tid; e < GH * (p.max_num_parts - k0); e += BT) {
            const int64_t off = (int64_t)(s * p.num_group + qg) * p.ml_ss + (int64_t)(h0 + e % GH) * p.ml_sh + k0 + e / GH;
            p.max_logits[off] = -INFINITY;
            p.exp_sums[off] = 0.0f;
        }
    };

    int64_t tsum = 0;
    int tmax = 0;
    for (int i = tid; i < p.num_seqs; i += BT) {
        const int Li = max(p.seq_lens[i], 0);
        tsum += Li;
        tmax = max(tmax, Li);
        if (w == 0 && Li == 0) {  // worker 0 covers the empty sequences, one thread each
            for (int e = 0; e < GH * p.max_num_parts; ++e) {
                const int64_t off = (int64_t)(i * p.num_group + qg) * p.ml_ss + (int64_t)(h0 + e % GH) * p.ml_sh + e / GH;
                p.max_logits[off] = -INFINITY;
                p.exp_sums[off] = 0.0f;
            }
        }
    }
    tsum = __shfl(wave_incl_sum_i64(tsum, lane), kWave - 1, kWave);
    tmax = wave_max_i32(tmax);
    if (lane == 0) {
        bal_w64[wave] = tsum;
        bal_w32[wave] = tmax;
    }
    __syncthreads();
    int64_t total_tokens = 0;
    int maxL = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        total_tokens += bal_w64[i];
        maxL = max(maxL, bal_w32[i]);
    }
    total_tokens = uniform_i64(total_tokens);
    maxL = __builtin_amdgcn_readfirstlane(maxL);
    __syncthreads();  // bal_w64 is reused by the scan below
    const int64_t W = p.num_workers;
    int64_t U = max((total_tokens + W - 1) / W, ((int64_t)maxL + p.max_num_parts - 2) / (p.max_num_parts - 1));
    U = max((U + 31) & ~int64_t(31), int64_t(32));
    if (total_tokens == 0 || (int64_t)w * U >= total_tokens) return;
    const int64_t r0 = (int64_t)w * U, r1 = min(r0 + U, total_tokens);

    // sequences in batches of BT: block scan of the lengths gives their
    // offsets; the ones meeting [r0, r1) form a contiguous run
    int64_t base = 0;
    for (int b0 = 0; b0 < p.num_seqs && base < r1; b0 += BT) {
        const int i = b0 + tid;
        const int Li = i < p.num_seqs ? max(p.seq_lens[i], 0) : 0;
        const int64_t inc = wave_incl_sum_i64(Li, lane);
        if (lane == kWave - 1) bal_w64[wave] = inc;
        if (tid == 0) {
            bal_first = BT;
            bal_last = -1;
        }
        __syncthreads();
        int64_t off = base + inc - Li, total = 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if (j < wave) off += bal_w64[j];
            total += bal_w64[j];
        }
        bal_off[tid] = off;
        bal_len[tid] = Li;
        if (Li > 0 && off < r1 && off + Li > r0) {
            atomicMin(&bal_first, tid);
            atomicMax(&bal_last, tid);
        }
        __syncthreads();
        const int first = __builtin_amdgcn_readfirstlane(bal_first);
        const int last = __builtin_amdgcn_readfirstlane(bal_last);
        total = uniform_i64(total);
        for (int j = first; j <= last; ++j) {
            const int64_t so = uniform_i64(bal_off[j]);
            const int Ls = __builtin_amdgcn_readfirstlane(bal_len[j]);
            if (Ls <= 0) continue;
            const int k = (int)(w - so / U);
            piece(b0 + j, k, (int)(max(r0, so) - so), (int)(min(r1, so + Ls) - so));
            if ((so + Ls - 1) / U == w) mark_empty(b0 + j, k + 1);  // this worker has the last piece
        }
        base += total;
        __syncthreads();  // bal_* are rewritten by the next batch
    }
}

bool decode_mla_supported(int dtype, int D, int Dv, int group, int block_size)
{
    return (dtype == PA_BF16 || dtype == PA_F16) && D == 576 && Dv == 512 && block_size == 1 &&
           (group == 64 || group == 128);
}

template <class E, int NW, bool ALIBI>
static void launch_mla_a(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    if (p.num_workers > 0)
        hipLaunchKernelGGL((k_decode_mla<E, NW, true, ALIBI>), dim3(p.num_workers, p.num_kv_heads * p.num_group, 1),
                           dim3(64 * NW), 0, st, p);
    else
        hipLaunchKernelGGL((k_decode_mla<E, NW, false, ALIBI>), dim3(num_seqs, p.num_kv_heads * p.num_group, parts),
                           dim3(64 * NW), 0, st, p);
}

template <class E, int NW>
static void launch_mla_nw(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    if (p.alibi) launch_mla_a<E, NW, true>(p, num_seqs, parts, st);
    else launch_mla_a<E, NW, false>(p, num_seqs, parts, st);
}

template <class E>
static hipError_t launch_mla_e(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    if (p.group == 128)
        launch_mla_nw<E, 4>(p, num_seqs, parts, st);
    else
        launch_mla_nw<E, 2>(p, num_seqs, parts, st);
    return hipGetLastError();
}

hipError_t launch_decode_mla(const DecodeParams& p, int dtype, int num_seqs, int parts, hipStream_t st)
{
    if (dtype == PA_BF16) return launch_mla_e<BF16>(p, num_seqs, parts, st);
    if (dtype == PA_F16) return launch_mla_e<F16>(p, num_seqs, parts, st);
    return hipErrorInvalidValue;
}

}  // namespace pa
