// common.h -- device helpers shared by the libpagedattn kernels (gfx950,
// 64-lane wavefronts). Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types. Storage is read as raw bits and widened to fp32.
// ---------------------------------------------------------------------------
struct F32 {
    using storage = float;
    static constexpr int size = 4;
    static constexpr int dtype = PA_F32;
};
struct F16 {
    using storage = _Float16;
    static constexpr int size = 2;
    static constexpr int dtype = PA_F16;
};
struct BF16 {
    using storage = __bf16;
    static constexpr int size = 2;
    static constexpr int dtype = PA_BF16;
};
// OCP FP8 E4M3 cache codes (caches only; dequantized with a scale)
struct FP8E4M3 {
    using storage = uint8_t;
    static constexpr int size = 1;
    static constexpr int dtype = PA_FP8_E4M3;
};

// E4M3 codes -> fp32 with gfx950's conversion (two codes, the low or high
// 16 bits of w, per instruction). It decodes OCP E4M3: sign, 4-bit exponent
// with bias 7, 3-bit mantissa, subnormals m * 2^-9, NaN for exponent 15 with
// mantissa 7, no infinities (checked for all 256 codes).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w, bool high)
{
    return high ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint8_t v)  // fp8 cache code
{
    const f32x2 f = e4m3x2_to_f32(v, false);
    return f[0];
}
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(__bf16 v)
{
    return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, v) << 16);
}

// ---------------------------------------------------------------------------
// Split partials (tmp_output). Phase 1 stores each split's normalised output
// converted to the workspace's element type (fp32, or f16 / bf16 rounded to
// nearest even); the type is uniform across a launch, so the branch on it is
// a scalar one. Phase 2 reads them back widened to fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 x = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 x = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, x);
}
// four consecutive values at element offset off; NT: nontemporal hint
template <bool NT = false>
__device__ __forceinline__ void store_tmp4(void* tmp, int dtype, int64_t off, f32x4 v)
{
    if (dtype == PA_F32) {
        f32x4* at = reinterpret_cast<f32x4*>(tmp) + (off >> 2);
        if constexpr (NT) __builtin_nontemporal_store(v, at);
        else *at = v;
    } else {
        const u32x2 w = dtype == PA_BF16 ? u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}
                                         : u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
        u32x2* at = reinterpret_cast<u32x2*>(tmp) + (off >> 2);
        if constexpr (NT) __builtin_nontemporal_store(w, at);
        else *at = w;
    }
}
__device__ __forceinline__ void store_tmp1(void* tmp, int dtype, int64_t off, float v)
{
    if (dtype == PA_F32)
        reinterpret_cast<float*>(tmp)[off] = v;
    else if (dtype == PA_BF16)
        reinterpret_cast<__bf16*>(tmp)[off] = (__bf16)v;
    else
        reinterpret_cast<_Float16*>(tmp)[off] = (_Float16)v;
}
// four consecutive partial values of element type E at p (4-element aligned)
template <class E>
__device__ __forceinline__ f32x4 load_tmp4(const typename E::storage* p)
{
    if constexpr (E::size == 4) {
        return *reinterpret_cast<const f32x4*>(p);
    } else {
        using S = typename E::storage;
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
        auto half = [&](int i) { return to_f32(__builtin_bit_cast(S, (uint16_t)(w[i >> 1] >> (16 * (i & 1))))); };
        return f32x4{half(0), half(1), half(2), half(3)};
    }
}

// Low / high 16-bit halves of a packed dword, widened.
template <class E> __device__ __forceinline__ float lo16(uint32_t w);
template <class E> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<BF16>(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
template <> __device__ __forceinline__ float hi16<BF16>(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo16<F16>(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi16<F16>(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Element i (0-based) of a 16-byte vector holding 16/size elements.
template <class E> __device__ __forceinline__ float elem16(const u32x4& v, int i)
{
    if constexpr (E::size == 1) {
        const f32x2 f = e4m3x2_to_f32(v[i >> 2], (i & 2) != 0);
        return (i & 1) ? f[1] : f[0];
    } else if constexpr (E::size == 4) {
        // copy the element out first: bit-casting the vector-element lvalue
        // directly reads element 0 with this compiler
        const uint32_t w = v[i];
        return __uint_as_float(w);
    } else {
        return (i & 1) ? hi16<E>(v[i >> 1]) : lo16<E>(v[i >> 1]);
    }
}

__device__ __forceinline__ u32x4 load16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load for cache data read once per step: the nontemporal hint
// keeps the lines from being allocated in L2 / the Infinity Cache, which
// measurably raises the HBM read rate of the paged gather on gfx950.
__device__ __forceinline__ u32x4 load16_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x2 load8_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

template <class E> __device__ __forceinline__ void store_out(void* base, int64_t idx, float v);
template <> __device__ __forceinline__ void store_out<F32>(void* base, int64_t idx, float v)
{
    reinterpret_cast<float*>(base)[idx] = v;
}
template <> __device__ __forceinline__ void store_out<F16>(void* base, int64_t idx, float v)
{
    reinterpret_cast<_Float16*>(base)[idx] = (_Float16)v;
}
template <> __device__ __forceinline__ void store_out<BF16>(void* base, int64_t idx, float v)
{
    reinterpret_cast<__bf16*>(base)[idx] = (__bf16)v;
}

// ---------------------------------------------------------------------------
// Page lists and the token -> (block, slot) map (block-table example of
// triton issue 2522; two-step gather of paged_attention_v2_triton.py).
// ---------------------------------------------------------------------------
struct PageList {
    const int32_t* pages;
    int64_t stride_s;  // row stride of a 2-D block table
    int64_t stride_b;  // element stride within a row (and CSR element stride)
    const int32_t* indptr;  // CSR row starts, or nullptr for a 2-D table
};

// First element of sequence s's page list.
__device__ __forceinline__ const int32_t* page_row(const PageList& pl, int s)
{
    int64_t off = pl.indptr ? (int64_t)pl.indptr[s] * pl.stride_b : (int64_t)s * pl.stride_s;
    return pl.pages + off;
}

// The two gather steps for token t (block_size = 1 << bs_shift): its page
// (physical block) pages[(t >> bs_shift) * stride_b], then its slot inside
// the block, t & (block_size - 1). Every decode kernel reads its block ids
// through page_of and takes slots with slot_of; the test hook
// paged_token_offsets() computes its offsets with the same two functions.
// P is int32_t* or the scalar-cache (constant address space) view of the
// same list.
template <class P>
__device__ __forceinline__ int32_t page_of(P row, int64_t stride_b, int64_t t, int bs_shift)
{
    return row[(t >> bs_shift) * stride_b];
}
__device__ __forceinline__ int64_t slot_of(int64_t t, int bs_shift)
{
    return t & ((int64_t(1) << bs_shift) - 1);
}

// Offset of token t: page * block_stride + slot * slot_stride.
__device__ __forceinline__ int64_t token_offset(const int32_t* row, int64_t stride_b, int64_t t,
                                                int bs_shift, int64_t block_stride,
                                                int64_t slot_stride)
{
    return (int64_t)page_of(row, stride_b, t, bs_shift) * block_stride + slot_of(t, bs_shift) * slot_stride;
}

// Split rule shared by phase 1 and phase 2: fixed partition size, or the
// per-sequence split count clamped to [1, max_parts] with the split length
// cdiv(L, n) rounded up to 64 tokens.
__device__ __forceinline__ int64_t split_length(int L, const int32_t* num_splits, int s,
                                                int partition_size, int max_parts)
{
    if (!num_splits) return partition_size;
    int n = num_splits[s];
    n = n < 1 ? 1 : (n > max_parts ? max_parts : n);
    int64_t Lc = L < 1 ? 1 : L;
    int64_t c = (Lc + n - 1) / n;
    return (c + 63) & ~int64_t(63);
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes).
// ---------------------------------------------------------------------------
// A 64-bit value that is the same in every lane, as a scalar (the compiler
// cannot tell that a value read from LDS is uniform).
__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Orders one wave's LDS writes before its later LDS reads (and the reads
// before later writes) without a workgroup barrier: a wave's LDS operations
// execute in order, so only the compiler must not move them across.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// Lane exchanges that stay in the vector ALU (no trip through the LDS
// crossbar a bpermute takes): DPP row permutations for partners inside a
// row of 16 lanes, the gfx950 permlane swaps for partners 16 and 32 lanes
// away. The reductions combine each lane with its partner in butterfly
// order, so every lane of the wave ends with the same bits.
namespace xlane {
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kHalfMirror = 0x141; // lane 7 - i within 8: lane ^ 4 once quads agree
constexpr int kMirror = 0x140;     // lane 15 - i within 16: lane ^ 8 once halves agree
}  // namespace xlane
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// op over lanes l and l ^ 16 (rows of 16 swapped pairwise), resp. l ^ 32.
template <class Op>
__device__ __forceinline__ float across16(float v, Op op)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
template <class Op>
__device__ __forceinline__ float across32(float v, Op op)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
struct MaxOp {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
    __device__ float operator()(float a, float b) const { return a + b; }
};
// Whole-wave reduction: DPP inside rows, then two bpermutes across rows.
// (The same reduction with the permlane swaps for the last two steps, all in
// the vector ALU, measured 20% slower in the one-token-per-lane kernel on
// 16-bit caches, with the loop's instruction mix unchanged; either half
// alone costs nothing, so the cross-row steps stay on the crossbar.)
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
    v = op(v, dpp_f32<xlane::kQuadXor1>(v));
    v = op(v, dpp_f32<xlane::kQuadXor2>(v));
    v = op(v, dpp_f32<xlane::kHalfMirror>(v));
    v = op(v, dpp_f32<xlane::kMirror>(v));
    v = op(v, __shfl_xor(v, 16, kWave));
    return op(v, __shfl_xor(v, 32, kWave));
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp{}); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, SumOp{}); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
