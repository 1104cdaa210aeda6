// decode_mla.hip -- phase 1 of split-KV decode for the MLA-style layout:
// many query heads (G = 64 or 128) over one latent kv head whose cache row
// holds both the key (all D values) and the value (its first Dv values),
// page size 1. What is computed is the phase-1 algorithm of
// paged_attention_v2_triton.py (module docstring: per split, scores
// q.K^T * scale, online softmax, weighted V; stores m, l and the normalised
// split output); the value rows are the leading Dv columns of the key rows,
// so every latent byte is read from HBM once per split.
//
// One 4-wave workgroup per (seq, kv head, head group of 64, split); wave w
// owns query heads 16w .. 16w+15 of its group (lane = 16*g + r, head r of
// the wave). At one wave per SIMD a wave keeps its heads' q (72 VGPRs) and
// accumulators (128) in registers. The split is walked in 16-token chunks:
//
//   staging  the chunk's 16 latent rows are copied HBM -> LDS by direct
//            global-to-LDS loads (no registers hold data in flight) into a
//            ring of NBUF chunk buffers, NBUF-1 chunks ahead. 16-byte piece
//            pc of row t sits at column pc ^ ((t >> 1) & 7) of its LDS row,
//            which spreads the 16 rows a QK operand read touches over
//            distinct LDS banks. Page ids of the split are staged in LDS.
//   QK       S^T[t][h] = sum_d K[t][d] Q[h][d]: v_mfma_f32_16x16x32 with the
//            chunk's 16 tokens as rows (A operand: one 16-byte piece of a K
//            row from LDS) and the wave's 16 heads as columns (B operand: q in
//            registers). Lane (g, r) receives tokens 4g..4g+3 of head r.
//   softmax  running max per head over the lane's 4 scores and the lanes r,
//            r+16, r+32, r+48; probabilities rounded to the cache type.
//   PV       O^T[dv][h] = sum_t V[t][dv] P[t][h]: v_mfma_f32_16x16x16 per 16
//            value columns. The B operand (P[4g..4g+3][r]) is what the softmax
//            left in lane (g, r); the A operand (V[4g..4g+3][16mt + r]) is a
//            column of the token-major rows, read with ds_read_b64_tr_b16:
//            within a 16-lane group, lane i receives value (i mod 4) of the
//            8-byte chunks addressed by lanes i/4 + 4j, so lane a addresses
//            row 4g + a/4, columns 16mt + 4(a%4) .. +3.
// Tokens past the split end are loaded from the last valid row (a real,
// finite row) and masked: scores -inf, probabilities 0.
#include <utility>

#include "kernels.h"

namespace pa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <class E> struct MlaOps;
template <> struct MlaOps<BF16> {
    typedef bf16x8 vec8;
    typedef __bf16 vec4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4 mma32(vec8 a, vec8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(vec4 a, vec4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                        __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
};
template <> struct MlaOps<F16> {
    typedef f16x8 vec8;
    typedef _Float16 vec4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4 mma32(vec8 a, vec8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(vec4 a, vec4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
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
// operations complete in issue order, so the read N places before the last
// one issued has landed; its value is threaded through the wait so nothing
// that uses it can be scheduled above it.
template <int N, class V>
__device__ __forceinline__ void lds_wait(V& v)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
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

// max of x over lanes l, l^16, l^32, l^48 (the four 16-lane rows)
__device__ __forceinline__ float row_max4(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS reads kept in flight ahead of their MFMAs (at most 15 can be
// outstanding per wave)
constexpr int kMlaReadAhead = 12;

// Largest divisor of `ins` that is at most `nw` (waves issuing the copies).
__host__ __device__ constexpr int loader_waves(int ins, int nw)
{
    int best = 1;
    for (int d = 1; d <= nw; ++d)
        if (ins % d == 0) best = d;
    return best;
}

constexpr int kMlaChunk = 16;    // tokens per chunk
constexpr int kMlaBuf = 6;       // chunk buffers in the LDS ring
constexpr int kMlaPageWin = 2048;  // page ids staged in LDS at a time

template <class E, int D, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void k_decode_mla(DecodeParams p)
{
    using T = typename E::storage;
    using Ops = MlaOps<E>;
    using vec8 = typename Ops::vec8;
    using vec4 = typename Ops::vec4;
    constexpr int CT = kMlaChunk;
    constexpr int PR = D * (int)sizeof(T) / 16;  // 16-byte pieces per latent row
    constexpr int INS = CT * PR / 64;              // copy instructions per chunk
    constexpr int LW = loader_waves(INS, NW);     // waves that issue copies
    constexpr int IPW = INS / LW;                 // copies per loader wave per chunk
    constexpr int KS = D / 32;                    // QK k-steps
    constexpr int MT = DV / 16;                   // PV value-column tiles
    constexpr int NB = kMlaBuf;
    static_assert(CT * PR % 64 == 0, "chunk must be a whole number of copy instructions");
    static_assert(PR % 8 == 0, "row pieces must be a multiple of 8 for the swizzle");
    static_assert(DV % 16 == 0 && DV <= D, "value columns are a prefix of the key row");

    __shared__ u32x4 ring[NB][CT * PR];
    __shared__ int32_t page_lds[kMlaPageWin];

    // grid (seq, kv head x head group, split): a workgroup serves 16*NW of
    // the kv head's G query heads; the head groups of one split read the
    // same latent rows, which the second reader finds in L2.
    const int ngroups = p.group / (16 * NW);
    const int s = blockIdx.x, kvh = blockIdx.y / ngroups, hg = blockIdx.y % ngroups, part = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const int h = kvh * p.group + hg * 16 * NW + wave * 16 + r;

    const int L = p.seq_lens[s];
    const int64_t len64 = split_length(L, p.num_splits, s, p.partition_size, p.max_num_parts);
    const int64_t start64 = (int64_t)part * len64;
    if (start64 >= (int64_t)L) {
        if (g == 0) {
            const int64_t mloff = (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
            p.max_logits[mloff] = -INFINITY;
            p.exp_sums[mloff] = 0.0f;
        }
        return;
    }
    const int start = (int)start64;
    const int end = (int)((int64_t)L < start64 + len64 ? (int64_t)L : start64 + len64);
    const int nc = (end - start + CT - 1) / CT;

    // B operand of QK: lane (g, r) holds q[h][32*ks + 8g .. +8]
    vec8 qv[KS];
    {
        const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)s * p.q_ss + (int64_t)h * p.q_sh + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qv[ks] = __builtin_bit_cast(vec8, load16(q + ks * 32));
    }

    const int32_t* row = page_row(p.pl, s);
    const int64_t sb = p.pl.stride_b;
    const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)kvh * p.k_sh;

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
            const T* src = kc + (int64_t)pg[j] * p.k_sb + (int64_t)((pc ^ ((t >> 1) & 7)) * 8);
            lds_copy16(src, dst + ins * 64);
        }
    };

    // Lazy rescaling: probabilities are taken against a reference max mref
    // that only moves when a chunk's max exceeds it by more than 2^8, so the
    // 128 accumulator values are rescaled rarely (p <= 256 meanwhile, well
    // inside fp32 / bf16 range). The true max is kept apart and (m, l) are
    // brought to it at the end, so the stored statistics are the exact
    // max logit and sum of exp(z - max).
    constexpr float kLazy = 8.0f;
    float mref = -INFINITY;  // reference max of head r (base 2)
    float mtrue = -INFINITY; // true running max of head r (base 2)
    float l = 0.0f;          // this lane's share of sum_t exp2(z_t - mref)
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // scores of chunk c for this lane's four tokens (base 2, masked past
    // the split end) and their max over the wave's tokens for head r
    auto scores = [&](int c, float (&sc)[4]) -> float {
        const int c0 = start + CT * c;
        const u32x4* buf = &ring[c % NB][0];
        // ---- scores. Piece (4ks + g) of row r sits at column (4ks + g) ^ rsw;
        // with rsw = 4*b + a' that is 4*(ks ^ b) + (g ^ a'), i.e. two base
        // addresses (even and odd k-steps) plus 128*(ks/2) as the immediate.
        // The 18 reads stream kMlaReadAhead ahead of their MFMAs, which
        // alternate between two accumulators to keep the matrix core fed.
        const uint32_t bufa = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)buf);
        const int rsw = (r >> 1) & 7;
        const uint32_t kbase = bufa + r * PR * 16 + 16 * (g ^ (rsw & 3));
        const uint32_t kb0 = kbase + 64 * (rsw >> 2);        // even k-steps
        const uint32_t kb1 = kbase + 64 * ((rsw >> 2) ^ 1);  // odd k-steps
        constexpr int RA = kMlaReadAhead < KS ? kMlaReadAhead : KS;
        u32x4 kr[KS];
        auto kread = [&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            kr[ks] = lds_read_b128<128 * (ks >> 1)>((ks & 1) ? kb1 : kb0);
        };
        static_for<RA>(kread);
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        static_for<KS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int issued = (i + RA < KS) ? i + RA : KS;
            lds_wait<issued - i - 1>(kr[i]);
            if constexpr (i & 1)
                s1 = Ops::mma32(__builtin_bit_cast(vec8, kr[i]), qv[i], s1);
            else
                s0 = Ops::mma32(__builtin_bit_cast(vec8, kr[i]), qv[i], s0);
            if constexpr (i + RA < KS) kread(std::integral_constant<int, i + RA>{});
            __builtin_amdgcn_sched_barrier(0);  // keep wait -> MFMA -> next read in order
        });
        const f32x4 sacc = s0 + s1;
        const int t0 = c0 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = (t0 + i < end) ? sacc[i] * p.scale_log2 : -INFINITY;
        return row_max4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    };

    // probabilities of chunk c against mref, and their weighted value rows
    auto weigh = [&](int c, const float (&sc)[4]) {
        const u32x4* buf = &ring[c % NB][0];
        // Value tile mt of this lane lives in piece 2mt + c1 (c1 = (r & 3) >> 1)
        // of row vrow, at column (2mt + c1) ^ vsw = 2*(mt ^ (vsw >> 1)) +
        // (c1 ^ (vsw & 1)): four base addresses (mt mod 4) plus 128*(mt/4)
        // as the immediate. The first reads are issued before the
        // probabilities are formed, so their latency overlaps that work.
        const uint32_t bufa = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)buf);
        const int vrow = 4 * g + (r >> 2);
        const int vsw = (vrow >> 1) & 7;
        const uint32_t vbase = bufa + vrow * PR * 16 + (r & 1) * 8 + 16 * ((((r & 3) >> 1)) ^ (vsw & 1));
        const int vx = vsw >> 1;
        const uint32_t vb4[4] = {vbase + 32 * (0 ^ vx), vbase + 32 * (1 ^ vx), vbase + 32 * (2 ^ vx),
                                 vbase + 32 * (3 ^ vx)};
        constexpr int RA = kMlaReadAhead < MT ? kMlaReadAhead : MT;
        s16x4 vr[MT];
        auto vread = [&](auto mtc) {
            constexpr int mt = decltype(mtc)::value;
            vr[mt] = lds_read_tr16<128 * (mt >> 2)>(vb4[mt & 3]);
        };
        static_for<RA>(vread);
        __builtin_amdgcn_sched_barrier(0);

        vec4 pv;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const T e = (T)fast_exp2(sc[i] - mref);
            pv[i] = e;
            psum += (float)e;
        }
        l += psum;
        // O^T[dv][h] += V^T[dv][t] P[t][h], one value tile per MFMA
        static_for<MT>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int issued = (i + RA < MT) ? i + RA : MT;
            lds_wait<issued - i - 1>(vr[i]);
            acc[i] = Ops::mma16(__builtin_bit_cast(vec4, vr[i]), pv, acc[i]);
            if constexpr (i + RA < MT) vread(std::integral_constant<int, i + RA>{});
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Ring pipeline: chunks c+1 .. c+NB-1 are in flight while chunk c is
    // used. Copies complete in issue order, so before chunk c a loader wave
    // waits until at most IPW copies per later chunk remain outstanding
    // (all of them in the last NB-2 chunks); the barrier then makes every
    // wave's copies visible and frees the slot chunk c-1 used, which the
    // copy of chunk c+NB-1 reuses.
    // q is in registers before the ring starts, so no wait inside the loop
    // has to cover its loads
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    for (int c = 0; c < NB - 1 && c < nc; ++c) issue(c);
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

    // The steady-state loop touches the accumulators only through MFMAs, so
    // they stay in accumulation registers across chunks; a chunk whose max
    // passes mref + kLazy leaves it, the accumulators are rescaled here
    // (every wave passes one barrier per chunk on either path), and the
    // loop resumes after that chunk.
    int c = 0;
    while (c < nc) {
        float sc[4];
        float mloc = -INFINITY;
        bool rescale = false;
        for (; c < nc; ++c) {
            advance(c);
            mloc = scores(c, sc);
            mtrue = fmaxf(mtrue, mloc);
            if (__builtin_amdgcn_ballot_w64(mloc > mref + kLazy)) {
                rescale = true;
                break;
            }
            weigh(c, sc);
        }
        if (!rescale) break;
        const float mn = fmaxf(mref, mloc);
        const float alpha = fast_exp2(mref - mn);  // 0 on the first chunk
        mref = mn;
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
        weigh(c, sc);
        ++c;
    }

    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int64_t mloff = (int64_t)s * p.ml_ss + (int64_t)h * p.ml_sh + part;
    if (g == 0) {
        p.max_logits[mloff] = mtrue * kLn2;
        p.exp_sums[mloff] = l * fast_exp2(mref - mtrue);
    }
    const float inv = 1.0f / l;
    float* out = p.tmp + (int64_t)s * p.tmp_ss + (int64_t)h * p.tmp_sh + (int64_t)part * p.tmp_sp + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(out + 16 * mt) = acc[mt] * inv;
}

bool decode_mla_supported(int dtype, int D, int Dv, int group, int block_size)
{
    return (dtype == PA_BF16 || dtype == PA_F16) && D == 576 && Dv == 512 && block_size == 1 &&
           (group == 64 || group == 128);
}

// One 4-wave workgroup (64 query heads) per head group: at 1 wave per SIMD a
// wave holds its 16 heads' q (72 VGPRs) and accumulators (128) with room to
// spare; with 8 waves (2 per SIMD) the same state spills.
constexpr int kMlaWaves = 4;

template <class E>
static hipError_t launch_mla_e(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    dim3 grid(num_seqs, p.num_kv_heads * (p.group / (16 * kMlaWaves)), parts);
    hipLaunchKernelGGL((k_decode_mla<E, 576, 512, kMlaWaves>), grid, dim3(64 * kMlaWaves), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_decode_mla(const DecodeParams& p, int dtype, int num_seqs, int parts, hipStream_t st)
{
    if (dtype == PA_BF16) return launch_mla_e<BF16>(p, num_seqs, parts, st);
    if (dtype == PA_F16) return launch_mla_e<F16>(p, num_seqs, parts, st);
    return hipErrorInvalidValue;
}

}  // namespace pa
