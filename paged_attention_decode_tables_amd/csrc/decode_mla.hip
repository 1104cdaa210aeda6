// decode_mla.hip -- phase 1 of split-KV decode for the MLA-style layout:
// many query heads (G = 64 or 128) over one latent kv head whose cache row
// holds both the key (all D = 576 values) and the value (its first Dv = 512
// values), page size 1. What is computed is the phase-1 algorithm of
// paged_attention_v2_triton.py (module docstring: per split, scores
// q.K^T * scale, online softmax, weighted V; stores m, l and the normalised
// split output); the value rows are the leading Dv columns of the key rows,
// so every latent byte is read from HBM once per split.
//
// One workgroup per (seq, kv head, split), or per balanced token range,
// serves all G heads with NW = G/32 waves, one per SIMD. The split is walked
// in 32-token chunks:
//
//   staging  the chunk's 32 latent rows are copied HBM -> LDS by direct
//            global-to-LDS loads (no registers hold data in flight, the
//            nontemporal hint on) into a ring of kMlaBuf chunk slots
//            (kMlaBuf64 at G = 64, so that two workgroups share a compute
//            unit), up to one fewer chunks ahead. A slot holds the rows' first 64 16-byte
//            pieces as 1 KB rows and their last 8 pieces as 128-byte rows
//            (see mla_fmain / mla_ftail for the bank swizzle), so each copy
//            instruction is one row from one page: wave w copies rows
//            TPW*w .. +TPW-1 with scalar base addresses. Page ids are read
//            by scalar loads, one chunk ahead.
//   QK       wave w, heads 32w .. 32w+31 (lane = 32*hl + c32, head c32):
//            S^T[t][h] = sum_d K[t][d] Q[h][d] on v_mfma_f32_32x32x16, the 32
//            tokens the rows (A operand: 16 bytes of a latent row from LDS),
//            the wave's 32 heads the columns (B operand: q in registers).
//            A-row m reads token perm(m) = 16*(m>>4) + 8*((m>>2)&1) +
//            4*((m>>3)&1) + (m&3), so with the accumulator layout (lane
//            32*hl + c32, register r: row 8*(r>>2) + 4*hl + (r&3), column
//            c32) lane (hl, c32) holds head c32's scores of tokens
//            16*(r>>3) + 8*hl + (r&7).
//   softmax  per head against a fixed reference (the split's first-chunk
//            max; see the kernel), probabilities rounded to the cache type
//            and written to an LDS buffer of [G heads][32 tokens].
//   PV       split by value columns: wave w owns column tiles NW*dt + w
//            for all G heads, O^T[dv][h] += V^T[dv][t] P[t][h] on
//            v_mfma_f32_32x32x16 per 32 columns, 32 heads and 16 tokens: A =
//            8 tokens of one value column (two ds_read_b64_tr_b16 of the
//            token-major rows: within a 16-lane group, lane i receives value
//            (i mod 4) of the 8-byte pieces addressed by lanes i/4 + 4j, so
//            lane a addresses row t0 + a/4, columns 4(a%4) .. +3 of its
//            16-column half), B = 16 bytes of the probability buffer. Each
//            wave reads a quarter of the chunk's value rows, and every
//            operand feeds four MFMAs.
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
    // two E4M3 codes (bytes 0-1 or, high, 2-3 of w) as two bf16 values
    static __device__ __forceinline__ uint32_t widen2(uint32_t w, bool high)
    {
        return high ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
                    : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    }
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct MlaOps<F16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ uint32_t widen2(uint32_t w, bool high)
    {
        return high ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
                    : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    }
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
// The nontemporal hint (the latent rows are read once per step) raises the
// copy stream's rate on the random 1152-byte rows (measured: 3.1 -> 3.6
// TB/s for the copies alone). The builtin only exists for the device pass
// (in the host pass it makes clang drop the kernel's launch stub), hence
// the guard.
__device__ __forceinline__ void lds_copy16(const void* src, __attribute__((address_space(3))) void* lds_dst)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int kNontemporal = 2;  // cache-policy bits: nt
    __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, kNontemporal);
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

// r == I ? a : b for a per-lane r and a uniform a, as a compare and a
// select: written as plain code, a chain of these over an array of page ids
// becomes a table in scratch memory indexed per lane.
template <int I>
__device__ __forceinline__ int select_eq(int r, int a, int b)
{
    int t;
    asm volatile("v_mov_b32 %1, %4\n\tv_cmp_eq_u32_e32 vcc, %2, %3\n\tv_cndmask_b32_e32 %0, %0, %1, vcc"
                 : "+v"(b), "=&v"(t)
                 : "n"(I), "v"(r), "s"(a)
                 : "vcc");
    return b;
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

// Ring layout of one chunk (32 latent rows): the first 64 16-byte pieces of
// every row (the 512 value columns, also the first 512 key columns) as a
// 1 KB row, then the last 8 pieces (the remaining key columns) of all 32
// rows as 128-byte rows. Piece pc of main row t sits at position pc ^
// mla_fmain(t), piece q of tail row t at q ^ mla_ftail(t) (XOR within groups
// of 16 and 8 pieces). LDS serves 256 B per clock, 16 lanes of a b128 access:
//  - QK reads (16 lanes: rows 0..15 or 16..31 at one piece) land on 16
//    distinct 16-byte bank groups since mla_fmain is a bijection on t & 15
//    and (t & 1, mla_ftail) one on t & 15;
//  - transposed P.V reads (32 lanes: rows 4u .. 4u+3, four consecutive
//    pieces each) since bits 2-3 of the XOR are t & 3 and bits 0-1
//    the same for the four rows.
// A main row is one copy instruction (64 lanes x 16 B) from one page: its
// page id is uniform, the lane's source piece is lane ^ mla_fmain(t).
__host__ __device__ constexpr int mla_fmain(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__host__ __device__ constexpr int mla_ftail(int t) { return (t >> 1) & 7; }

#ifndef PA_MLA_BUF
#define PA_MLA_BUF 4
#endif
#ifndef PA_MLA_KAHEAD
#define PA_MLA_KAHEAD 8
#endif
constexpr int kMlaChunk = 32;             // tokens per chunk
constexpr int kMlaBuf = PA_MLA_BUF;       // chunk slots in the LDS ring
#ifndef PA_MLA_BUF8
#define PA_MLA_BUF8 4
#endif
constexpr int kMlaBuf8 = PA_MLA_BUF8;     // fp8 caches: chunk slots of fp8 rows in the copy ring
// G = 64 (two waves): two chunk slots, so that two workgroups fit in a
// compute unit's LDS and all four SIMDs work (one chunk in flight each)
#ifndef PA_MLA_BUF64
#define PA_MLA_BUF64 2
#endif
constexpr int kMlaBuf64 = PA_MLA_BUF64;
// G = 64 over fp8 caches: two fp8 slots and one widened slot (widened at the
// start of each chunk), for the same two workgroups a compute unit
constexpr int kMlaBuf8x64 = 2;
constexpr int kMlaKAhead = PA_MLA_KAHEAD; // QK operand reads in flight ahead of their MFMAs
constexpr int kMlaHeadsPerWave = 32;
// Balanced splits: virtual tokens charged for each piece a worker starts
// (measured: a piece costs about 20 us beyond its chunks on the MLA batch,
// the time of ~250 tokens).
constexpr int kMlaPieceCharge = 256;

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

// s_waitcnt lgkmcnt(N), with the value operand of the next MFMAs (and, for
// the first value operand of a k-step, its probability operands) threaded
// through it, so that nothing using them is scheduled above the wait.
template <int N, class B>
__device__ __forceinline__ void lds_wait_v(B& b0, B& b1)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(b0), "+v"(b1) : "n"(N));
}
template <int N, class A, class B>
__device__ __forceinline__ void lds_wait_pv(A (&a)[4], B& b0, B& b1)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%6)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b0), "+v"(b1)
                 : "n"(N));
}
template <int N, class A, class B>
__device__ __forceinline__ void lds_wait_pv(A (&a)[2], B& b0, B& b1)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(b0), "+v"(b1) : "n"(N));
}
// Workgroup barrier that orders LDS accesses only: this wave's LDS
// operations are complete, then s_barrier. __syncthreads() also fences
// global memory, i.e. waits for every outstanding store and copy; under a
// saturated memory system that is a full round trip (several microseconds)
// each time, for ordering nothing here needs.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// max of three scores (they are never NaN: no quieting needed)
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
template <int OFF>
__device__ __forceinline__ void lds_write_b128(uint32_t lds_addr, u32x4 v)
{
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(lds_addr), "v"(v), "n"(OFF) : "memory");
}

// Two probabilities rounded to the cache type, packed, and their sum.
template <class E> struct MlaPack;
template <> struct MlaPack<BF16> {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ uint32_t pack(float a, float b, float& sum)
    {
        const v2 x = {(__bf16)a, (__bf16)b};
        const v2 one = {(__bf16)1.0f, (__bf16)1.0f};
        sum = __builtin_amdgcn_fdot2_f32_bf16(x, one, sum, false);
        return __builtin_bit_cast(uint32_t, x);
    }
};
template <> struct MlaPack<F16> {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ uint32_t pack(float a, float b, float& sum)
    {
        const v2 x = {(_Float16)a, (_Float16)b};
        const v2 one = {(_Float16)1.0f, (_Float16)1.0f};
        sum = __builtin_amdgcn_fdot2(x, one, sum, false);
        return __builtin_bit_cast(uint32_t, x);
    }
};

// P.V operand schedule of one chunk (per wave): 2 k-steps of 16 tokens, each
// with HT probability operands (one b128 read of the P buffer each) and DT
// value operands (two transposed reads each), read in that order; MFMA m =
// (kk, dt, ht), ht fastest, needs value operand (kk, dt) and everything
// read before it. Reads are issued as far ahead as 15 outstanding LDS
// operations (the lgkmcnt limit) allow.
template <int HT, int DT> struct PvSchedule {
    static constexpr int kReads = 2 * (HT + DT);   // operand reads (P: 1 op, V: 2 ops)
    static constexpr int kMfma = 2 * DT * HT;
    // LDS operations up to and including read r
    static constexpr int ops_through(int r)
    {
        int n = 0;
        for (int i = 0; i <= r; ++i) n += (i % (HT + DT)) < HT ? 1 : 2;
        return n;
    }
    // read index that MFMA m needs last: value operand (kk, dt)
    static constexpr int need(int m)
    {
        const int kk = m / (DT * HT), dt = (m / HT) % DT;
        return kk * (HT + DT) + HT + dt;
    }
    // last read issued before MFMA m: all that fit in 15 outstanding operations
    // once the reads MFMA m-1 needed have landed
    static constexpr int issued(int m)
    {
        const int done = m == 0 ? -1 : need(m - 1);
        const int base = done < 0 ? 0 : ops_through(done);
        int r = done;
        while (r + 1 < kReads && ops_through(r + 1) - base <= 15) ++r;
        return r;
    }
    static constexpr int wait(int m) { return ops_through(issued(m)) - ops_through(need(m)); }
};

// ---- balanced splits: the sequences' tokens in sequence order, each
// non-empty sequence preceded by kMlaPieceCharge virtual tokens (the cost of
// starting a piece: loading its query and the first chunks, storing its
// partial output), total T'; worker w (the XCD-grouped rank of blockIdx.x) takes virtual positions
// [w*U, (w+1)*U), so a worker that starts a sequence inside its range gets
// that many fewer real tokens. piece(s, slot, start, end) runs one piece of
// sequence s for the workgroup's GH heads h0 .. h0+GH-1 (query token qg).
template <int NW, class Piece>
__device__ __forceinline__ void mla_balanced(const DecodeParams& p, const int qg, const int h0, const int GH,
                                             Piece&& piece)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    constexpr int BT = 64 * NW;
    constexpr int C = kMlaPieceCharge;
    __shared__ int64_t bal_w64[NW];
    __shared__ int bal_w32[NW];
    __shared__ int64_t bal_off[BT];
    __shared__ int bal_len[BT];
    __shared__ int bal_first, bal_last;
    const int tid = threadIdx.x;
    // Token range of this workgroup. Workgroups are dealt to the 8 XCDs
    // round robin by linear id; with W a multiple of 8, XCD x runs ranges
    // x*W/8 .. (x+1)*W/8 - 1, so neighbouring ranges (mostly of one
    // sequence) share that XCD's L2 for their query (latent-row batch: HBM
    // reads 1.148x -> 1.045x the cache bytes). Any other W: identity.
    const int w = (gridDim.x & 7) == 0 ? (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3)
                                       : (int)blockIdx.x;
    // m = -inf, l = 0 in slots [k0, max_num_parts) of sequence s, all heads
    // here (all threads of the workgroup together)
    auto mark_empty = [&](int s, int k0) {
        for (int e = tid; e < GH * (p.max_num_parts - k0); e += BT) {
            const int64_t off = (int64_t)(s * p.num_group + qg) * p.ml_ss + (int64_t)(h0 + e % GH) * p.ml_sh + k0 + e / GH;
            p.max_logits[off] = -INFINITY;
            p.exp_sums[off] = 0.0f;
        }
    };

    // With at most BT sequences every thread loads its length once and keeps
    // it for the scan below (one memory round trip for the whole schedule).
    const bool one_round = p.num_seqs <= BT;
    int Lmine = 0;
    int64_t tsum = 0;
    int tmax = 0;
    for (int i = tid; i < p.num_seqs; i += BT) {
        const int Li = max(p.seq_lens[i], 0);
        if (i == tid) Lmine = Li;
        tsum += Li > 0 ? Li + C : 0;
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
    lds_barrier();
    int64_t total_virtual = 0;
    int maxL = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        total_virtual += bal_w64[i];
        maxL = max(maxL, bal_w32[i]);
    }
    total_virtual = uniform_i64(total_virtual);
    maxL = __builtin_amdgcn_readfirstlane(maxL);
    lds_barrier();  // bal_w64 is reused by the scan below
    const int64_t W = p.num_workers;
    int64_t U = max((total_virtual + W - 1) / W, ((int64_t)maxL + p.max_num_parts - 2) / (p.max_num_parts - 1));
    U = max((U + 31) & ~int64_t(31), int64_t(32));
    if (total_virtual == 0 || (int64_t)w * U >= total_virtual) return;
    const int64_t r0 = (int64_t)w * U, r1 = min(r0 + U, total_virtual);

    // sequences in batches of BT: a block scan of the virtual lengths gives
    // their virtual offsets; the ones meeting [r0, r1) form a contiguous run
    int64_t base = 0;
    for (int b0 = 0; b0 < p.num_seqs && base < r1; b0 += BT) {
        const int i = b0 + tid;
        const int Li = one_round ? Lmine : (i < p.num_seqs ? max(p.seq_lens[i], 0) : 0);
        const int Vi = Li > 0 ? Li + C : 0;
        const int64_t inc = wave_incl_sum_i64(Vi, lane);
        if (lane == kWave - 1) bal_w64[wave] = inc;
        if (tid == 0) {
            bal_first = BT;
            bal_last = -1;
        }
        lds_barrier();
        int64_t off = base + inc - Vi + C, total = 0;  // virtual position of the sequence's first token
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
        lds_barrier();
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
        lds_barrier();  // bal_* are rewritten by the next batch
    }
}

// ALIBI: scores carry the slopes' bias (a separate instance, so the plain
// kernel keeps its registers).
// BAL = false: one workgroup per (seq, kv head, split) of the fixed or
// per-sequence split rule. BAL = true: balanced splits, one workgroup per
// (token range, kv head).
template <class E, int NW, bool BAL, bool ALIBI, bool KV8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_decode_mla(DecodeParams p)
{
    using T = typename E::storage;
    using Ops = MlaOps<E>;
    using vec8 = typename Ops::vec8;
    constexpr int D = 576, DV = 512;
    constexpr int CT = kMlaChunk;
    constexpr int PR = D * (int)sizeof(T) / 16;  // 16-byte pieces per latent row (72)
    constexpr int MP = 64;                        // pieces of a main row (1 KB)
    constexpr int TP = PR - MP;                   // pieces of a tail row (8)
    constexpr int TAIL = CT * MP * 16;            // byte offset of the tail rows in a slot
    constexpr int TPW = CT / NW;                  // rows each wave copies
    constexpr int IPW = TPW + TPW * TP / 64;      // copy instructions per wave per chunk
    constexpr int KS = D / 16;                    // QK k-steps
    constexpr int P8 = D / 16;                    // 16-byte pieces of an fp8 latent row (36)
    constexpr int IP8 = (TPW * P8 + 63) / 64;     // fp8 copy instructions per wave per chunk
    constexpr int NB = KV8 ? (NW == 2 ? kMlaBuf8x64 : kMlaBuf8) : NW == 2 ? kMlaBuf64 : kMlaBuf;  // chunk slots of the copy ring
    constexpr int NUSE = KV8 ? (NW == 2 ? 1 : 2) : 0;  // fp8: slots of widened rows
    constexpr int IPC = KV8 ? IP8 : IPW;          // copy instructions per wave per chunk
    constexpr int HPW = kMlaHeadsPerWave;
    constexpr int G = HPW * NW;                   // heads of the workgroup
    constexpr int HT = NW;                        // P.V head tiles: all G heads
    constexpr int DT = DV / 32 / NW;              // P.V value-column tiles of one wave
    using Sched = PvSchedule<HT, DT>;
    static_assert(PR == MP + 8 && TPW % 8 == 0, "ring layout: 64 + 8 pieces a row, tail rows 8 to a copy");
    static_assert(KS % 4 == 0 && DT % 2 == 0, "tiling");
    static_assert(IPC * (NB - 2) <= 63, "vmcnt is a 6-bit field");
    static_assert(!KV8 || NUSE == 1 || NB >= 3, "fp8: chunk c+1 is widened while chunk c is in use");

    // The copy ring: NB slots of CT rows. Caches of the query's type are
    // copied straight into the layout QK and P.V read (see mla_fmain); fp8
    // rows land as copied (576-byte rows) and each wave widens its rows of
    // chunk c+1, during chunk c, into the other of two slots in that layout
    // (G = 64: its rows of chunk c into the one slot, at the chunk's start).
    constexpr int SLOT = CT * PR, SLOT8 = CT * P8;  // u32x4 words of a slot
    __shared__ __attribute__((aligned(256))) u32x4 ring[KV8 ? NUSE * SLOT + NB * SLOT8 : NB * SLOT];
    // LDS byte addresses: the slot QK and P.V read for chunk c, the slot its
    // copies land in
    auto use_slot = [](int c) -> uint32_t {
        return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)&ring[KV8 ? (NUSE == 2 ? (c & 1) * SLOT : 0) : (c % NB) * SLOT]);
    };
    auto copy_slot = [](int c) -> uint32_t {
        return (uint32_t)(uintptr_t)((
            __attribute__((address_space(3))) const char*)&ring[KV8 ? NUSE * SLOT + (c % NB) * SLOT8 : (c % NB) * SLOT]);
    };
    __shared__ u32x4 pbuf[G * 4];  // probabilities of a chunk: [head][32 tokens] of T, 64 B a head
    __shared__ int rerun_flag;

    const int ngroups = p.group / G;
    const int hg = blockIdx.y % ngroups, kq = blockIdx.y / ngroups;
    // query token qg of every sequence (rows s * num_group + qg)
    const int qg = kq % p.num_group, kvh = kq / p.num_group;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, c32 = lane & 31, hl = lane >> 5;
    const int h0 = kvh * p.group + hg * G;  // first head of the workgroup
    const int h = h0 + wave * HPW + c32;

    // One split (or balanced piece): tokens [start, end) of sequence s, its
    // statistics and normalised output stored in split slot `part`.
    auto piece = [&](const int s, const int part, const int start, const int end) {
    lds_barrier();  // the previous piece's LDS reads are done
    // With balanced splits the pieces run in a loop. The lane and head
    // indices are then re-derived through an opaque zero, so the compiler
    // cannot hoist what depends on them out of that loop: kept live across
    // it, they pushed the loop over chunks past the register file (spills
    // in it cost a quarter of the kernel's time).
    int opaque = 0;
    if constexpr (BAL) asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
    const int lane = (int)(threadIdx.x & 63) + opaque, c32 = lane & 31, hl = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) + opaque;  // scalar
    const int h = h0 + opaque + wave * HPW + c32;  // this lane's head in QK and the softmax
    const int nc = (end - start + CT - 1) / CT;

    // B operand of QK: lane (hl, c32) holds q[h][16*ks + 8*hl .. +8]. With a
    // negative scale the query is negated (exact) and |scale| used, so the
    // largest raw score is the largest logit.
    const float scale = fabsf(p.scale_log2);
    const uint32_t qflip = p.scale_log2 < 0.0f ? 0x80008000u : 0u;
    vec8 qv[KS];
    {
        const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)(s * p.num_group + qg) * p.q_ss + (int64_t)h * p.q_sh + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w = load16(q + ks * 16);
            w ^= qflip;
            qv[ks] = __builtin_bit_cast(vec8, w);
        }
    }

    // the sequence's page list, read through the scalar data cache: every
    // page id a wave needs is uniform across it
    typedef __attribute__((address_space(4))) const int32_t* cptr;
    const int64_t sb = p.pl.stride_b;
    const int64_t roff = p.pl.indptr ? (int64_t)((cptr)(uintptr_t)p.pl.indptr)[s] * sb : (int64_t)s * p.pl.stride_s;
    const cptr rowc = (cptr)(uintptr_t)(p.pl.pages + roff);
    const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)kvh * p.k_sh;
    // ALiBi: head h's slope in base-2 units. Scores then grow toward the end
    // of the sequence, so a split usually passes the first chunk's reference
    // by more than the headroom and runs twice.
    const int L = ALIBI ? p.seq_lens[s] : 0;
    const float slope = ALIBI ? p.alibi[h] * kLog2e : 0.0f;

    // page ids of the rows this wave copies for chunk c (rows past the split
    // end take the last valid row's page: real data, masked later)
    auto load_pages = [&](int c, int32_t (&pg)[TPW]) {
        const int r0 = start + CT * c + TPW * wave;
        if (sb == 1 && r0 + TPW <= end) {  // consecutive ids, all before the split end: wide loads
#pragma unroll
            for (int j = 0; j < TPW; ++j) pg[j] = page_of(rowc, 1, r0 + j, 0);
        } else {
#pragma unroll
            for (int j = 0; j < TPW; ++j) pg[j] = page_of(rowc, sb, min(r0 + j, end - 1), 0);
        }
    };

    // copy chunk `c` (tokens start + CT*c ...) into ring slot c % NB: wave w
    // copies rows TPW*w .. TPW*w + TPW-1, one instruction per main row (a
    // scalar base address) and one per 8 tail rows; fp8 rows as 16-byte
    // pieces, 64 consecutive pieces of the wave's rows an instruction (a
    // lane's row is one of the 3 an instruction can touch).
    auto issue = [&](int c, const int32_t (&pg)[TPW]) {
        // an opaque zero: the lane offsets below are recomputed per chunk (one
        // XOR a copy) rather than hoisted out of the chunk loop, where they
        // would take 20 registers and be spilled
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        if constexpr (KV8) {
            const uint8_t* kc8 = reinterpret_cast<const uint8_t*>(p.kc) + (int64_t)kvh * p.k_sh;
            const uint32_t base = copy_slot(c) + 16 * TPW * P8 * wave;
            static_for<IP8>([&](auto kc_) {
                constexpr int k = decltype(kc_)::value;
                constexpr int r0 = 64 * k / P8;  // first row an instruction touches
                const int i = 64 * k + lane + z;  // piece of the wave's rows
                const int rl = i / P8, q = i - rl * P8;
                int pgl = pg[r0];
                if constexpr (r0 + 1 < TPW) pgl = select_eq<r0 + 1>(rl, pg[r0 + 1], pgl);
                if constexpr (r0 + 2 < TPW) pgl = select_eq<r0 + 2>(rl, pg[r0 + 2], pgl);
                const uint8_t* src = kc8 + (int64_t)pgl * p.k_sb + 16 * q;
                if (64 * k + 64 <= TPW * P8 || i < TPW * P8)
                    lds_copy16(src, (__attribute__((address_space(3))) void*)(uintptr_t)(base + 1024 * k));
            });
            return;
        }
        const uint32_t lane16 = (uint32_t)(lane * 16 + z);
        const uint32_t slot = copy_slot(c);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = TPW * wave + j;
            const char* rowp = reinterpret_cast<const char*>(kc + (int64_t)pg[j] * p.k_sb);
            lds_copy16(rowp + (lane16 ^ (uint32_t)(16 * mla_fmain(t))),
                       (__attribute__((address_space(3))) void*)(uintptr_t)(slot + t * MP * 16));
        }
#pragma unroll
        for (int k = 0; k < TPW / 8; ++k) {
            const int t0 = TPW * wave + 8 * k, r = (lane + z) >> 3, t = t0 + r, q = (lane + z) & 7;
            int pgl = pg[8 * k];  // the page of this lane's row
#pragma unroll
            for (int i = 1; i < 8; ++i) pgl = r == i ? pg[8 * k + i] : pgl;
            const T* src = kc + (int64_t)pgl * p.k_sb + 8 * (MP + (q ^ mla_ftail(t)));
            lds_copy16(src, (__attribute__((address_space(3))) void*)(uintptr_t)(slot + TAIL + t0 * TP * 16));
        }
    };

    // Fixed reference: probabilities are taken against mref, head h's max
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
    //
    // ALiBi (bf16): the bias slope * position grows along the split, by at
    // most shift = slope * (end - 1 - start) (base 2) past any first-chunk
    // token, so the reference starts at the first chunk's max + shift and a
    // split reruns only when its scores grow by more than that plus the
    // headroom. If the true max ends more than kUnder below the reference,
    // the split also reruns (against the true max): otherwise a token flushed
    // to zero (below mref - 126) would be one within 126 - kUnder of the true
    // max. With kUnder = 64 every flushed token weighs < 2^-62 of the largest.
    constexpr float kHeadroom = std::is_same<E, F16>::value ? 15.0f : 64.0f;
    constexpr bool kShift = ALIBI && std::is_same<E, BF16>::value;
    constexpr float kUnder = 64.0f;
    const float shift = kShift && slope > 0.0f ? slope * (float)(end - 1 - start) : 0.0f;
    float mref = -INFINITY;  // reference max of head h (base 2)
    float mtrue = -INFINITY; // true running max of head h (base 2)
    float l = 0.0f;          // this lane's share of sum_t exp2(z_t - mref), rounded p
    bool over = false;       // a score of head h passed mref + kHeadroom
    f32x16 acc[DT][HT];      // O^T[value column][head] of this wave's columns, all G heads
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[dt][ht][i] = 0.0f;

    // QK operand addresses: A-row c32 reads ring row perm(c32), piece
    // 2*ks + hl. For ks < 32 that is main-row position 16*(ks>>3) + ((2*(ks&7)
    // + hl) ^ fmain): eight base addresses (ks mod 8) plus 256*(ks/8) as the
    // immediate; for ks >= 32 tail position (2*(ks-32) + hl) ^ ftail: four
    // bases.
    const int trow = 16 * (c32 >> 4) + 8 * ((c32 >> 2) & 1) + 4 * ((c32 >> 3) & 1) + (c32 & 3);
    uint32_t kb_main[8], kb_tail[4];
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) kb_main[k8] = trow * MP * 16 + 16 * ((2 * k8 + hl) ^ mla_fmain(trow));
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) kb_tail[k4] = TAIL + trow * TP * 16 + 16 * ((2 * k4 + hl) ^ mla_ftail(trow));
    // P.V value operands (A = V^T[32 value columns][16 tokens]) of column
    // tile mt = NW*dt + wave (the wave's tiles interleave with the others'):
    // transposed read (kk, rd) covers rows t = 16kk + 8hl + 4rd + a/4 (a =
    // lane & 15) and value columns 32mt + 16*g16 + 4*(a&3) .. +3 (g16 = (lane
    // >> 4) & 1), i.e. piece pc = 4mt + 2*g16 + ((a&3) >> 1), 8 bytes in when
    // a is odd. With fmain(t) = 4*(a/4) + 2hl + rd, position pc ^ fmain(t) has
    // bits 0-1 (2*g16 + ((a&3) >> 1)) ^ 2hl ^ rd, bits 2-3 (mt & 3) ^ a/4 and
    // bits 4-5 mt >> 2: lane bases for rd = 0, 1 and (NW*dt) & 3 (0, or 0 and
    // 2 when NW = 2), plus kk*16 KB + rd*4 KB + 256*(mt >> 2) as the immediate.
    uint32_t vb_lane[2][2];
    {
        const int a = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
#pragma unroll
            for (int x = 0; x < 2; ++x)
                vb_lane[rd][x] = (8 * hl + (a >> 2)) * MP * 16 + 64 * (((2 * x) | wave) ^ (a >> 2)) +
                                 16 * ((2 * g16 + ((a & 3) >> 1)) ^ (2 * hl) ^ rd) + 8 * (a & 1);
    }
    // P buffer: head j's 32 probabilities are one 64-byte row, tokens 8i ..
    // 8i+7 in 16-byte piece i ^ ((j >> 2) & 3), so the 16 lanes of one b128
    // access (16 heads, one piece) cover distinct banks. Lane (hl, c32)
    // writes head 32*wave + c32's pieces hl and 2 + hl (its tokens) and, for
    // P.V head tile ht, reads head 32*ht + c32's piece 2kk + hl (B operand:
    // tokens 16kk + 8hl .. +7).
    const uint32_t pbase = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)&pbuf[0]);
    const int psw = (c32 >> 2) & 3;
    const uint32_t pa0 = pbase + c32 * 64 + 16 * (hl ^ psw);        // piece hl
    const uint32_t pa1 = pbase + c32 * 64 + 16 * ((hl ^ psw) ^ 2);  // piece 2 + hl
    const uint32_t pw0 = pa0 + 2048 * wave, pw1 = pa1 + 2048 * wave;

    // raw scores S^T[t][h] of chunk c: lane (hl, c32) gets head h's scores of
    // tokens 16*(r>>3) + 8*hl + (r&7), r = 0..15
    auto qk = [&](int c) -> f32x16 {
        const uint32_t bufa = use_slot(c);
        constexpr int RA = kMlaKAhead < KS ? kMlaKAhead : KS;
        u32x4 kr[KS];
        auto kread = [&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            if constexpr (ks < 32)
                kr[ks] = lds_read_b128<256 * (ks >> 3)>(bufa + kb_main[ks & 7]);
            else
                kr[ks] = lds_read_b128<0>(bufa + kb_tail[ks - 32]);
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
        return sacc;
    };

    // probabilities of chunk c against mref, rounded to the cache type and
    // written to the P buffer; TAILC: the chunk at the split end, whose
    // tokens from nvalid on are masked (every other chunk is full)
    auto softmax = [&](int c, const f32x16& sacc, auto tailc) {
        constexpr bool TAILC = decltype(tailc)::value;
        const int c0 = start + CT * c;
        const int nvalid = end - c0;  // >= 1
        float z[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 16 * (r >> 3) + 8 * hl + (r & 7);
            if constexpr (ALIBI)
                z[r] = sacc[r] * scale + slope * (float)(c0 + t - (L - 1));
            else
                z[r] = sacc[r];
            if constexpr (TAILC) z[r] = t < nvalid ? z[r] : -INFINITY;
        }
        float mx = max3f(z[0], z[1], z[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = max3f(mx, z[r], z[r + 1]);
        mx = fmaxf(mx, z[15]);
        float mloc = across32(mx, MaxOp{});  // token 0 is valid, so lane half 0 has a finite score
        if constexpr (!ALIBI) mloc *= scale;
        mref = mref == -INFINITY ? mloc + shift : mref;
        over |= mloc > mref + kHeadroom;
        mtrue = fmaxf(mtrue, mloc);
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            e[r] = fast_exp2(ALIBI ? z[r] - mref : fmaf(z[r], scale, -mref));
            if constexpr (TAILC) e[r] = 16 * (r >> 3) + 8 * hl + (r & 7) < nvalid ? e[r] : 0.0f;
        }
        u32x4 w0, w1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w0[i] = MlaPack<E>::pack(e[2 * i], e[2 * i + 1], l);
            w1[i] = MlaPack<E>::pack(e[8 + 2 * i], e[8 + 2 * i + 1], l);
        }
        lds_write_b128<0>(pw0, w0);
        lds_write_b128<0>(pw1, w1);
    };

    // O^T[this wave's value columns][all G heads] += V^T P over chunk c
    auto pv = [&](int c, auto after_reads) {
        const uint32_t slot = use_slot(c);
        u32x4 pr[2][HT];
        s16x4 vr[2][DT][2];
        // read r of the schedule: (kk, P operand ht) or (kk, value operand dt)
        auto read = [&](auto rc) {
            constexpr int r = decltype(rc)::value;
            constexpr int kk = r / (HT + DT), i = r % (HT + DT);
            if constexpr (i < HT) {
                pr[kk][i] = lds_read_b128<2048 * i>(kk ? pa1 : pa0);
            } else {
                constexpr int dt = i - HT;
                constexpr int x = ((NW * dt) & 3) >> 1;  // (NW*dt) & 3 is 0 or 2
                constexpr int imm = kk * 16 * MP * 16 + 256 * ((NW * dt) >> 2);
                vr[kk][dt][0] = lds_read_tr16<imm>(slot + vb_lane[0][x]);
                vr[kk][dt][1] = lds_read_tr16<imm + 4 * MP * 16>(slot + vb_lane[1][x]);
            }
        };
        static_for<Sched::kMfma>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int kk = m / (DT * HT), dt = (m / HT) % DT, ht = m % HT;
            constexpr int from = m == 0 ? 0 : Sched::issued(m - 1) + 1;
            static_for<Sched::issued(m) + 1 - from>([&](auto jc) {
                read(std::integral_constant<int, from + decltype(jc)::value>{});
            });
            // a wait before the first MFMA of each value operand (the
            // probability operands of the k-step were read before it)
            if constexpr (ht == 0) {
                if constexpr (dt == 0)
                    lds_wait_pv<Sched::wait(m)>(pr[kk], vr[kk][dt][0], vr[kk][dt][1]);
                else
                    lds_wait_v<Sched::wait(m)>(vr[kk][dt][0], vr[kk][dt][1]);
            }
            const u32x4 a = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[kk][dt][0], vr[kk][dt][0], 0, 1)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[kk][dt][0], vr[kk][dt][0], 2, 3)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[kk][dt][1], vr[kk][dt][1], 0, 1)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(vr[kk][dt][1], vr[kk][dt][1], 2, 3))};
            acc[dt][ht] = Ops::mma(__builtin_bit_cast(vec8, a), __builtin_bit_cast(vec8, pr[kk][ht]), acc[dt][ht]);
            __builtin_amdgcn_sched_barrier(0);
            // every read of the chunk has landed: scalar loads issued here
            // cannot hold up a counted LDS wait
            if constexpr (m == Sched::kMfma - HT) {
                after_reads();
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };

    // Ring pipeline: chunks c+1 .. c+NB-1 are in flight while chunk c is
    // used. Copies complete in issue order, so before chunk c a loader wave
    // waits until at most IPW copies per later chunk remain outstanding
    // (all of them in the last NB-2 chunks); the barrier then makes every
    // wave's copies visible, and, since every wave has finished chunk c-1,
    // frees its ring slot and the P buffer. The slot is refilled with chunk
    // c+NB-1 later in chunk c, just before the barrier that publishes the
    // probabilities: a wave that reaches that barrier early waits there
    // anyway, so the time its copies take to issue is mostly hidden (the
    // latent-row batch: 123.4 -> 121.1 us against issuing them right after
    // the first barrier).
    int32_t pg_next[TPW];  // page ids of the next chunk to copy
    // fp8: widen this wave's rows of chunk c (its own copies, landed) into
    // the use slot, bit-exact (E4M3 values are bf16 and f16 values)
    auto widen = [&](int c) {
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const int ln = lane + z;
        const uint32_t src = copy_slot(c) + 16 * TPW * P8 * wave + 16 * ln;
        const uint32_t dst = use_slot(c);
        u32x4 w[IP8];
        static_for<IP8>([&](auto kc_) {
            constexpr int k = decltype(kc_)::value;
            w[k] = lds_read_b128<1024 * k>(src);
        });
        lds_wait<0>(w[0]);
        static_for<IP8>([&](auto kc_) {
            constexpr int k = decltype(kc_)::value;
            const int i = 64 * k + ln;
            if (64 * k + 64 <= TPW * P8 || i < TPW * P8) {
                const int rl = i / P8, q = i - rl * P8, t = TPW * wave + rl;
                u32x4 lo, hi;  // values 0-7 and 8-15 of the piece's 16 codes
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t a = MlaOps<E>::widen2(w[k][d], false), b = MlaOps<E>::widen2(w[k][d], true);
                    if (d < 2) {
                        lo[2 * d] = a;
                        lo[2 * d + 1] = b;
                    } else {
                        hi[2 * d - 4] = a;
                        hi[2 * d - 3] = b;
                    }
                }
                uint32_t a0, a1;  // byte addresses of the two widened pieces
                if (q < MP / 2) {
                    a0 = dst + t * MP * 16 + 16 * ((2 * q) ^ mla_fmain(t));
                    a1 = dst + t * MP * 16 + 16 * ((2 * q + 1) ^ mla_fmain(t));
                } else {
                    const int tq = 2 * (q - MP / 2);
                    a0 = dst + TAIL + t * TP * 16 + 16 * (tq ^ mla_ftail(t));
                    a1 = dst + TAIL + t * TP * 16 + 16 * ((tq + 1) ^ mla_ftail(t));
                }
                lds_write_b128<0>(a0, lo);
                lds_write_b128<0>(a1, hi);
            }
        });
    };
    auto advance = [&](int c) {
        if (c + NB - 2 < nc)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(IPC * (NB - 2)));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        // A plain s_barrier (see lds_barrier): the copies this barrier
        // publishes are covered by the explicit wait above; the compiler
        // fences keep LDS accesses on their side of the barrier.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (KV8 && NUSE == 1) {
            // the barrier above: every wave is done with chunk c-1 in the slot
            widen(c);
            lds_barrier();  // every wave's rows of chunk c are widened
        }
    };
    // fp8: widen this wave's rows of chunk c+1 into the other use slot (every
    // wave finished chunk c-1, its last reader, before chunk c's first
    // barrier), once its copies have landed: at most the copies of the
    // chunks after it, up to c+NB-2, are still outstanding. The next
    // barrier publishes the rows; it is one fewer barrier a chunk than
    // widening chunk c at its start, and early waves do it while they would
    // wait at the probability barrier anyway.
    auto widen_next = [&](int c) {
        if (c + 1 >= nc) return;
        if (c + NB - 2 < nc)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(IPC * (NB - 3)));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        widen(c + 1);
    };
    // refill the slot freed at chunk c's first barrier; then every wave's
    // probabilities of the chunk (and, fp8, its widened rows of chunk c+1)
    // are in LDS
    auto p_ready = [&](int c) {
        if constexpr (KV8 && NUSE == 2) widen_next(c);
        if (c + NB - 1 < nc) issue(c + NB - 1, pg_next);
        lds_barrier();
    };
    // one pass over the split
    auto run = [&]() {
        for (int c = 0; c < NB - 1 && c < nc; ++c) {
            int32_t pg[TPW];
            load_pages(c, pg);
            issue(c, pg);
        }
        if (NB - 1 < nc) load_pages(NB - 1, pg_next);
        // One memory round trip for the query, the first chunks and the
        // previous piece's stores; no wait inside the loop covers them.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        if constexpr (KV8 && NUSE == 2) widen(0);  // published by chunk 0's first barrier
        for (int c = 0; c < nc; ++c) {
            advance(c);
            const f32x16 sacc = qk(c);
            if (end - start - CT * c < CT)
                softmax(c, sacc, std::true_type{});
            else
                softmax(c, sacc, std::false_type{});
            p_ready(c);
            pv(c, [&]() {
                if (c + NB < nc) load_pages(c + NB, pg_next);
            });
        }
    };

    if (threadIdx.x == 0) rerun_flag = 0;
    run();
    if (over || (kShift && mtrue < mref - kUnder)) rerun_flag = 1;  // benign race: every writer stores 1
    lds_barrier();
    if (rerun_flag) {  // uniform across the workgroup
        mref = mtrue;
        l = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[dt][ht][i] = 0.0f;
        lds_barrier();  // every wave is done with the ring
        run();
    }
    lds_barrier();  // every wave is done with the P buffer

    // statistics of head h; every wave needs the sums of all G heads
    l = across32(l, SumOp{});
    float* lsum = reinterpret_cast<float*>(&pbuf[0]);
    const int64_t mloff = (int64_t)(s * p.num_group + qg) * p.ml_ss + (int64_t)h * p.ml_sh + part;
    if (hl == 0) {
        lsum[wave * HPW + c32] = l;
        p.max_logits[mloff] = mtrue * kLn2;
        p.exp_sums[mloff] = l * fast_exp2(mref - mtrue);
    }
    lds_barrier();
    // lane (hl, c32), register 4i + j of tile (dt, ht) holds value column
    // 32*(NW*dt + wave) + 8i + 4hl + j of head 32ht + c32
    const int64_t out = (int64_t)(s * p.num_group + qg) * p.tmp_ss + (int64_t)(h0 + c32) * p.tmp_sh +
                        (int64_t)part * p.tmp_sp + 32 * wave + 4 * hl;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float inv = p.v_scale / lsum[32 * ht + c32];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store_tmp4(p.tmp, p.tmp_dtype, out + (int64_t)(32 * ht) * p.tmp_sh + 32 * NW * dt + 8 * i,
                           f32x4{acc[dt][ht][4 * i], acc[dt][ht][4 * i + 1], acc[dt][ht][4 * i + 2],
                                 acc[dt][ht][4 * i + 3]} * inv);
    }
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

    mla_balanced<NW>(p, qg, h0, HPW * NW, piece);
}

bool decode_mla_supported(int dtype, int D, int Dv, int group, int block_size)
{
    return (dtype == PA_BF16 || dtype == PA_F16) && D == 576 && Dv == 512 && block_size == 1 &&
           (group == 64 || group == 128);
}

template <class E, int NW, bool ALIBI, bool KV8>
static void launch_mla_k(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    if (p.num_workers > 0)
        hipLaunchKernelGGL((k_decode_mla<E, NW, true, ALIBI, KV8>),
                           dim3(p.num_workers, p.num_kv_heads * p.num_group, 1), dim3(64 * NW), 0, st, p);
    else
        hipLaunchKernelGGL((k_decode_mla<E, NW, false, ALIBI, KV8>),
                           dim3(num_seqs, p.num_kv_heads * p.num_group, parts), dim3(64 * NW), 0, st, p);
}

template <class E, int NW, bool ALIBI>
static void launch_mla_a(const DecodeParams& p, int num_seqs, int parts, hipStream_t st)
{
    if (p.kv_fp8) launch_mla_k<E, NW, ALIBI, true>(p, num_seqs, parts, st);
    else launch_mla_k<E, NW, ALIBI, false>(p, num_seqs, parts, st);
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
