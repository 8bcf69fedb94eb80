// gdn2_device.h -- device-side building blocks for the gfx950 (CDNA4) kernels:
// element types, MFMA fragments, LDS fragment loads and small helpers.
//
// MFMA tiles are 16x16 with fp32 accumulators.  A "fragment" holds the 32
// contraction slots one K-step of a 16x16 output consumes, 8 per lane: lane l
// covers output row/column (l % 16) and slot group g = l / 16, elements
// e = 0..7.  For bf16 operands one v_mfma_f32_16x16x32_bf16 consumes the 8
// elements at once; for fp32 operands eight v_mfma_f32_16x16x4_f32 consume one
// element each.  Either way the product sums over all 32 (g, e) slots, so the
// loader may map slots to contraction indices in any order, as long as both
// operands use the same map.  Two maps are used:
//   contiguous : slot (g, e) -> 8g + e                    (both operands from LDS)
//   permuted   : slot (g, e) -> 4g + e (e < 4), 16 + 4g + e - 4 (e >= 4)
// The permuted map is exactly where a 16x16 fp32 accumulator keeps its rows
// (lane l holds rows 4g..4g+3 of column l % 16), so an accumulator pair that
// covers 32 rows is directly a B operand, without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- element conversion -------------------------------------------------
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// ---- fragments ------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// single fp32 MFMA step (16x16x4)
__device__ __forceinline__ void mma_f32x4(f32x4& acc, float a, float b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// K = 16 steps: lane l covers row/column l % 16 and contraction slots 4g + e, e = 0..3.  An
// accumulator (lane holds rows 4g..4g+3) is directly a K = 16 B operand in this map.
template <typename T> struct Frag16;
template <> struct Frag16<bf16> { bf16x4 v; };
template <> struct Frag16<float> { float v[4]; };
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mma16(f32x4& acc, const Frag16<bf16>& a, const Frag16<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a.v),
                                                    __builtin_bit_cast(s16x4, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag16<float>& a, const Frag16<float>& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}
// four contiguous elements (p aligned to 4 * sizeof(T))
__device__ __forceinline__ Frag16<bf16> load16(const bf16* p) {
    Frag16<bf16> f;
    f.v = *reinterpret_cast<const bf16x4*>(p);
    return f;
}
__device__ __forceinline__ Frag16<float> load16(const float* p) {
    Frag16<float> f;
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = x[e];
    return f;
}
template <typename T> __device__ __forceinline__ Frag16<T> frag16_from_acc(const f32x4& a);
template <> __device__ __forceinline__ Frag16<bf16> frag16_from_acc<bf16>(const f32x4& a) {
    Frag16<bf16> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = (bf16)a[e];
    return f;
}
template <> __device__ __forceinline__ Frag16<float> frag16_from_acc<float>(const f32x4& a) {
    Frag16<float> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = a[e];
    return f;
}

// contiguous map: p points at element [row][kbase + 8g]; needs 16-byte alignment
__device__ __forceinline__ Frag<bf16> load_contig(const bf16* p) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
}
__device__ __forceinline__ Frag<float> load_contig(const float* p) {
    Frag<float> f;
    f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[e + 4] = hi[e]; }
    return f;
}

// permuted map: p points at element [row][kbase + 4g]; needs 8-byte alignment (bf16)
__device__ __forceinline__ Frag<bf16> load_perm(const bf16* p) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
    Frag<bf16> f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
}
__device__ __forceinline__ Frag<float> load_perm(const float* p) {
    f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    f32x4 hi = *reinterpret_cast<const f32x4*>(p + 16);
    Frag<float> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[e + 4] = hi[e]; }
    return f;
}

// B operand from two accumulators covering contraction rows [0,16) and [16,32)
template <typename T> __device__ __forceinline__ Frag<T> frag_from_acc(const f32x4& lo, const f32x4& hi);
template <> __device__ __forceinline__ Frag<bf16> frag_from_acc<bf16>(const f32x4& lo, const f32x4& hi) {
    Frag<bf16> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = (bf16)lo[e]; f.v[e + 4] = (bf16)hi[e]; }
    return f;
}
template <> __device__ __forceinline__ Frag<float> frag_from_acc<float>(const f32x4& lo, const f32x4& hi) {
    Frag<float> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[e + 4] = hi[e]; }
    return f;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// N consecutive elements through vector loads (p aligned to 16 bytes or to N * sizeof(T),
// whichever is smaller)
template <typename T, int N> struct Vec { T v[N]; };
template <typename T, int N>
__device__ __forceinline__ Vec<T, N> load_vec(const T* p) {
    Vec<T, N> r;
    if constexpr (N == 1) {
        r.v[0] = *p;
    } else {
        typedef T V __attribute__((ext_vector_type(N)));
        constexpr int AL = N * (int)sizeof(T) < 16 ? N * (int)sizeof(T) : 16;
        const V x = *reinterpret_cast<const V*>(__builtin_assume_aligned(p, AL));
#pragma unroll
        for (int i = 0; i < N; ++i) r.v[i] = x[i];
    }
    return r;
}

// exp(x) for x <= 0 through the hardware base-2 exponential
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// 1 / (1 + e^-x) through the hardware base-2 exponential and reciprocal (about 1 ulp each); for
// x below about -88, e^-x overflows to infinity and the reciprocal of infinity is the limit 0
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// How a forward kernel takes the per-token decay and the two gates (page "Why NVIDIA Gated
// DeltaNet-2 separates erase and write gates", axbrief.com, section "Gated Delta Rule-2": b and
// w are sigmoids of projections of the token; the decay takes the same form, alpha = sigmoid(a)).
//   GatesActivated: log alpha in fp32, b and w as given;
//   GatesLogits:    the projections' outputs a, xb, xw in the input dtype, activated on load
//                   (alpha = sigmoid(a), b = sigmoid(xb), w = sigmoid(xw)), so no activated copy
//                   of them is ever stored.
struct GatesActivated {
    using Decay = float;
    // the decay input of a token that decays nothing (alpha = 1)
    __device__ static __forceinline__ Decay no_decay() { return 0.f; }
    // a decay input of zero decays nothing: a token read as zeros is the identity
    static constexpr bool zero_is_identity = true;
    __device__ static __forceinline__ float alpha(float log_alpha) { return exp_neg(log_alpha); }
    __device__ static __forceinline__ float gate(float g) { return g; }
};
struct GatesLogits {
    using Decay = bf16;
    __device__ static __forceinline__ Decay no_decay() { return (bf16)__builtin_inff(); }
    static constexpr bool zero_is_identity = false;  // sigmoid(0) = 1/2
    __device__ static __forceinline__ float alpha(float a) { return sigmoid_f(a); }
    __device__ static __forceinline__ float gate(float x) { return sigmoid_f(x); }
};


// Packed sequences, longest first.  A launch walks its ns sequences in workgroup order, one
// chain of chunks per (sequence, head, slice); when the lengths differ, a long sequence that
// starts late sets the launch's length.  So sequence slot r (in dispatch order) takes the
// r-th longest sequence, ties in index order.  Lengths are the offsets clamped into
// [0, Tparam] as the kernels clamp them.  Every thread of the workgroup calls this, before
// anything else uses LDS; scratch must hold kMaxSort + 1 ints: the lengths in [0, ns) and the
// selected sequence at index kMaxSort (every caller's LDS block asserts that size).  For
// ns > kMaxSort, slot r takes sequence r and scratch is not touched.
constexpr int kMaxSort = 512;
__device__ __forceinline__ int longest_first(const int64_t* __restrict__ cu, int ns, int r, int Tparam, int* scratch) {
    if (ns > kMaxSort) return r;
    for (int i = threadIdx.x; i < ns; i += blockDim.x) {
        const int64_t lo = min(max(cu[i], (int64_t)0), (int64_t)Tparam);
        const int64_t hi = min(max(cu[i + 1], lo), (int64_t)Tparam);
        scratch[i] = (int)(hi - lo);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < ns; i += blockDim.x) {
        const int li = scratch[i];
        int rank = 0;
        for (int j = 0; j < ns; ++j) {
            const int lj = scratch[j];
            rank += (lj > li) || (lj == li && j < i);
        }
        if (rank == r) scratch[kMaxSort] = i;  // ranks are a permutation: one writer
    }
    __syncthreads();
    const int sel = scratch[kMaxSort];
    __syncthreads();
    return sel;
}

}  // namespace gdn2
