// gdn2_chunk_bwd.hip -- backward pass (vector-Jacobian product) of the chunked GDN-2
// recurrence on gfx950.
//
// Page "Why NVIDIA Gated DeltaNet-2 separates erase and write gates" (axbrief.com), section
// "Gated Delta Rule-2": the backward pass cannot reuse Kimi Delta Attention's scalar
// shortcut, because the erase and the write side carry different diagonal gates, so the gate
// factors sit inside the inner products that accumulate the gradients; the pages derive the
// vector-Jacobian product with the gates in it.  Here it is derived for the chunk form of the
// forward (C = 64).  Per chunk, with S the state entering it, G the chunk-local cumulative
// log-decay (per key channel), Gamma = e^G, kh = b.k, KG = kh.Gamma, QG = q.Gamma and
// KR = k.Gamma_C / Gamma:
//
//     U = T (w.v - KG S),   O = QG S + P U,   S' = Gamma_C.S + KR^T U,   T = (I + A)^{-1}.
//
// Given dO and dS' (the gradient of the state leaving the chunk):
//
//     dU  = P^T dO + KR dS',   dR = T^T dU            (dR: gradient of w.v - KG S)
//     dS  = Gamma_C.dS' + QG^T dO - KG^T dR           (the state entering the chunk)
//     dv  = dR.w,   dw = dR.v
//     dA  = -dR U^T (j < i),   dP = dO U^T (j <= i)
//     dq  = Gamma.(dO S^T)  + sum_j dP_ij k_j Gamma_{i<-j}
//     dkh = Gamma.(-dR S^T) + sum_j dA_ij k_j Gamma_{i<-j}
//     dk  = (Gamma_C / Gamma).(U dS'^T) + sum_i (dA_ij kh_i + dP_ij q_i) Gamma_{i<-j} + b.dkh
//     db  = k.dkh
//
// Every decay factor is e^{G_i - G_j} with q, kh on the i side and k on the j side, so the
// gradient of G_i is q.dq + kh.dkh - k.(dk - b.dkh) = q.dq + 2 kh.dkh - k.dk; G_C = G_63 adds
// sum_i KR_i.(U dS'^T)_i + Gamma_C.diag(dS' S^T).  The gradient of log alpha is the reverse
// cumulative sum of these over the chunk.
//
// Four launches:
//   0. bwd_local_kernel, every chunk independently: the chunk-local quantities in fp32 (A and
//      P from the inputs, T = (I + A)^{-1}, W = T KG, U0 = T (w.v), KR, QG, Gamma_C), one record
//      per chunk;
//   1. bwd_fwd_kernel, one workgroup per (sequence, head, slice of value columns): the forward
//      re-run from the records, U = U0 - W S and S' = Gamma_C.S + KR^T U, storing the state
//      entering every chunk and U;
//   2. bwd_state_kernel, one workgroup per (sequence, head, slice): the chunks in reverse order
//      with dS in MFMA accumulators, dS = Gamma_C.dS' + QG^T dO - W^T dU (KG^T T^T = W^T);
//      stores dS' of every chunk, dR, and dS of the first chunk (the gradient of the initial
//      state);
//   3. bwd_chunk_kernel, runs of consecutive chunks of one (sequence, head) per workgroup:
//      every gradient of each chunk's inputs, independently of the other chunks; the next
//      chunk's first loads are in flight during the current chunk's last phase.
// Precision: with fp32 inputs every product runs on fp32 MFMA (v_mfma_f32_16x16x4_f32); with
// bf16 inputs the chunk-local kernel keeps fp32 MFMA, and the products of kernels 1-3 take bf16
// hi/lo operands (three v_mfma_f32_16x16x32_bf16 per product, about 16 significant bits per
// operand).  Accumulation is fp32 throughout.
//
// Decays in kernels 0 and 3: a chunk whose whole-chunk decay stays >= e^-40 on every channel
// pivots all factors at the chunk start (k / Gamma is then finite, and every masked product is
// one MFMA pass); any other chunk forms its masked sums element by element from
// e^{G_i - G_j}, which never exceeds 1.
#include <type_traits>

#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {
namespace bw {

constexpr int C = 64;
constexpr int NT = 512;                  // 8 waves
constexpr float kMildLog = -40.f;        // whole-chunk log-decay bound of the pivoted form
constexpr float kLog2e = 1.4426950408889634f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads, so a prefetch stays in flight across it (no thread reads global memory that
// another thread of the kernel writes).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A value the compiler cannot see through: lane indices made opaque at the top of every chunk
// keep the chunk loop's address arithmetic inside the loop (hoisted out of it, the addresses
// outnumber the registers and are spilled to scratch).
__device__ __forceinline__ int opq(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Materialises x here: the compiler may not sink its computation past this point (a value
// still being computed when a reload of the registers it reads is issued keeps the old and the
// new value live together, and the loop then copies a register that a load has not filled yet,
// which waits for every memory operation in flight).
__device__ __forceinline__ void pin(f32x4& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x4 mfma4(const f32x4& acc, float a, float b) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}
// e^x for any x (overflow to inf and underflow to 0 as the hardware exponential does)
__device__ __forceinline__ float exp_any(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Decay exponents.  The element phase splits a chunk into blocks of L tokens; Gl_i is the
// cumulative log alpha from the start of token i's block, and OFF[b] the sum over the blocks
// before b, kept as an unevaluated hi + lo pair (two-sum), so that
//     G_i - G_j = (Gl_i - Gl_j) + (OFF[bi] - OFF[bj])
// is formed from numbers no larger than one block's sum, and the suffix sum G_C - G_i =
// (block sum - Gl_i) + (sum over the later blocks) without a difference of two large sums.
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// NTILE independent 16 x 16 products over the same contraction length K (compile time), with
// the steps of all tiles interleaved, so that the MFMA chains of different tiles hide each
// other's latency: acc[t] += sum_k A(t, m, k) B(t, k, n).  Within each block of 16 along k,
// lane group g4 supplies k = k0 + 4 g4 + s at step s (the sum is the same in any order), so a
// lane's four steps read four consecutive k: with k the contiguous index of both operands in
// LDS, that is one 16-byte read per operand and block.
template <int NTILE, int K, class FA, class FB>
__device__ __forceinline__ void mm_n(f32x4 (&acc)[NTILE], FA A, FB B, int l16, int g4) {
    // one block of 16 at a time: deeper unrolling lets the compiler hoist more operand loads
    // than the register file holds
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += 16) {
        float a[4][NTILE], b[4][NTILE];
#pragma unroll
        for (int t = 0; t < NTILE; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                a[s][t] = A(t, l16, k0 + 4 * g4 + s);
                b[s][t] = B(t, k0 + 4 * g4 + s, l16);
            }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < NTILE; ++t) acc[t] = mfma4(acc[t], a[s][t], b[s][t]);
    }
}

// bf16 hi/lo operands: x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi) and |r| <= 2^-17 |x|;
// a product takes hi.hi + hi.lo + lo.hi (the dropped lo.lo is below 2^-16 relative), three
// v_mfma_f32_16x16x32_bf16 for what costs eight v_mfma_f32_16x16x4_f32 per 32 k in fp32.
__device__ __forceinline__ void split_hl(const f32x4& x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int z = 0; z < 4; ++z) {
        hi[z] = (bf16)x[z];
        lo[z] = (bf16)(x[z] - (float)hi[z]);
    }
}
// As mm_n over hi/lo operand planes, K a multiple of 32: lane group g4 supplies k0 + 8 g4 + e
// (e = 0..7) of each block of 32; A(t, m, k, plane) and B(t, k, n, plane) point at the 8
// contiguous bf16 of k .. k + 7 (plane 0 hi, 1 lo).
template <int NTILE, int K, class FA, class FB>
__device__ __forceinline__ void mm_hl(f32x4 (&acc)[NTILE], FA A, FB B, int l16, int g4) {
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += 32) {
        bf16x8 ah[NTILE], al[NTILE], bh[NTILE], bl[NTILE];
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
            ah[t] = *reinterpret_cast<const bf16x8*>(A(t, l16, k0 + 8 * g4, 0));
            al[t] = *reinterpret_cast<const bf16x8*>(A(t, l16, k0 + 8 * g4, 1));
            bh[t] = *reinterpret_cast<const bf16x8*>(B(t, k0 + 8 * g4, l16, 0));
            bl[t] = *reinterpret_cast<const bf16x8*>(B(t, k0 + 8 * g4, l16, 1));
        }
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], bh[t], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], bl[t], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[t], bh[t], acc[t], 0, 0, 0);
    }
}

__device__ __forceinline__ f32x4 mf16(const f32x4& acc, const bf16x4& a, const bf16x4& b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), acc,
                                                     0, 0, 0);
}
__device__ __forceinline__ f32x4 mf32(const f32x4& acc, const bf16x8& a, const bf16x8& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// hi/lo of eight values
__device__ __forceinline__ void split_hl8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int z = 0; z < 8; ++z) {
        hi[z] = (bf16)x[z];
        lo[z] = (bf16)(x[z] - (float)hi[z]);
    }
}

// p advanced by a byte offset: with p uniform across the wave and the offset a 32-bit per-lane
// value, the access takes a scalar base and one vector register for the address
template <typename T>
__device__ __forceinline__ T* at_byte(T* p, uint32_t off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + off);
}
template <typename T>
__device__ __forceinline__ const T* at_byte(const T* p, uint32_t off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + off);
}

// Writes a wave's split units of one 16-key column block into its LDS tile of token rows,
// [2][C][LD] bf16 (hi plane, then lo): U[u][pl] holds tokens 8 (g4 + 4 u) .. + 7 of key l16.
// The lanes of each even/odd pair (keys 2m and 2m + 1) swap half of their tokens through a
// DPP quad permutation, so that a lane writes four-byte key pairs (tokens 0..3 of its unit from
// the even lane, 4..7 from the odd one) instead of two-byte elements.  Every lane of the wave
// must be active.
template <int LD>
__device__ __forceinline__ void stage_key_pairs(bf16* tile, const bf16x8 (&U)[2][2], int l16, int g4) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const bool odd = l16 & 1;
    const int m = l16 >> 1;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
            const u32x4 w = __builtin_bit_cast(u32x4, U[u][pl]);  // word k: tokens 2k (low), 2k + 1
            unsigned* dst = reinterpret_cast<unsigned*>(tile + pl * C * LD + (8 * (g4 + 4 * u) + 4 * odd) * LD) + m;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const unsigned mine = odd ? w[2 + q] : w[q];
                const unsigned give = odd ? w[q] : w[2 + q];
                const unsigned got = (unsigned)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
                const unsigned lo = odd ? got : mine, hi = odd ? mine : got;  // keys 2m, 2m + 1
                dst[(2 * q) * (LD / 2)] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                dst[(2 * q + 1) * (LD / 2)] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
            }
        }
}

// Eight packed bf16 values split at n: the first n (n clamped to 0..8) in `first`, the others
// in `rest`, zeros elsewhere (bit masks on the two 16-bit halves of each 32-bit word)
__device__ __forceinline__ void take_first(const bf16x8& x, int n, bf16x8& first, bf16x8& rest) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_bit_cast(u32x4, x);
    u32x4 m;
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = (2 * q < n ? 0xffffu : 0u) | (2 * q + 1 < n ? 0xffff0000u : 0u);
    first = __builtin_bit_cast(bf16x8, v & m);
    rest = __builtin_bit_cast(bf16x8, v & ~m);
}

// This thread's L tokens of key channel c in the element phase, every load issued at once: a
// token past the end reads the last token, and the caller zeroes it.
template <typename In, int L>
struct KeyIn {
    float g[L];
    In q[L], k[L], b[L];
};
// tokens t0 .. t0 + L - 1 (the last token past the end) of channel ch; base and t0 uniform
// across the wave, so each load takes a scalar row address and the lane's channel offset
template <typename In, int L>
__device__ __forceinline__ void load_key(KeyIn<In, L>& in, const In* __restrict__ q, const In* __restrict__ k,
                                         const In* __restrict__ b, const float* __restrict__ g, int64_t base,
                                         int ch, int64_t rk, int t0, int T) {
#pragma unroll
    for (int m = 0; m < L; ++m) {
        const int64_t o = base + (int64_t)min(t0 + m, T - 1) * rk;
        in.g[m] = *at_byte(g + o, (uint32_t)ch * 4u);
        in.q[m] = *at_byte(q + o, (uint32_t)ch * (uint32_t)sizeof(In));
        in.k[m] = *at_byte(k + o, (uint32_t)ch * (uint32_t)sizeof(In));
        in.b[m] = *at_byte(b + o, (uint32_t)ch * (uint32_t)sizeof(In));
    }
}

// N consecutive floats (N = 2 or 4) as one access
template <int N>
__device__ __forceinline__ void load_n(float (&d)[N], const float* p) {
    if constexpr (N == 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = x[i];
    } else {
        static_assert(N == 2, "width");
        const float2 x = *reinterpret_cast<const float2*>(p);
        d[0] = x.x;
        d[1] = x.y;
    }
}
template <int N>
__device__ __forceinline__ void store_n(float* p, const float (&d)[N]) {
    if constexpr (N == 4) {
        *reinterpret_cast<f32x4*>(p) = f32x4{d[0], d[1], d[2], d[3]};
    } else {
        static_assert(N == 2, "width");
        *reinterpret_cast<float2*>(p) = make_float2(d[0], d[1]);
    }
}

// ---------------------------------------------------------------------------------------
// Kernel 0: the chunk-local quantities, every chunk independently (a workgroup walks a run of
// consecutive chunks of one sequence and head, loading the next chunk's inputs one chunk
// ahead).  Each chunk gets one fp32 record (layout in gdn2_launch.h): T = (I + A)^{-1}, P,
// W = T KG, KR, QG, U0 = T (w.v) and Gamma_C.
// ---------------------------------------------------------------------------------------
// Record layout.  W, KR and U0 row-major ([token][channel]); T, P, QG and second copies of W
// and KR swizzled for reads of one channel over 16 tokens per lane: entry (token i, channel c)
// of a 64 x n matrix sits at sw(i, c) = [c / 16][i / 16][i mod 4][c mod 16][(i / 4) mod 4],
// so that lane (g, n16) of a wave reads the tokens 16 j4 + 4 x + g (x = 0..3) of channel
// 16 b + n16 as one 16-byte unit, and the 64 lanes' units for one j4 are contiguous.
__host__ __device__ constexpr int sw(int i, int c) {
    return ((((c >> 4) * 4 + (i >> 4)) * 4 + (i & 3)) * 16 + (c & 15)) * 4 + ((i >> 2) & 3);
}
// With bf16 inputs the products over tokens in the serial passes take bf16 hi/lo operands, so
// T, QG and the second copies of W and KR are stored split: a hi and a lo plane of bf16
// (64 n elements apart, the fp32 matrix's bytes), entry (token i, channel c) at element
// hl_unit(i, c) * 8 + i mod 8 of each, hl_unit = [c / 16][i / 32][(i / 8) mod 4][c mod 16]:
// lane (g, n16) reads the tokens 32 b + 8 g .. 32 b + 8 g + 7 of channel 16 cb + n16 as one
// 16-byte unit per plane.
__host__ __device__ constexpr int hl_unit(int i, int c) {
    return (((c >> 4) * 2 + (i >> 5)) * 4 + ((i >> 3) & 3)) * 16 + (c & 15);
}
// eight consecutive tokens' values, split, to unit u of the planes at base (npl elements apart)
__device__ __forceinline__ void put_hl8(bf16* base, int npl, int u, const float (&x)[8]) {
    bf16x8 h, l;
    split_hl8(x, h, l);
    *reinterpret_cast<bf16x8*>(base + u * 8) = h;
    *reinterpret_cast<bf16x8*>(base + npl + u * 8) = l;
}
template <int DK, int DV>
struct Rec {
    static constexpr int64_t OT = 0, OP = C * C, OW = 2 * C * C, OWS = OW + C * DK, OKR = OWS + C * DK,
                             OKRS = OKR + C * DK, OQG = OKRS + C * DK, OU0 = OQG + C * DK, OGC = OU0 + C * DV;
    static constexpr int64_t SIZE = bwd_rec_floats(DK, DV);
    static_assert(OGC + DK <= SIZE && SIZE % 64 == 0, "record layout");
};

template <typename In, int DK, int DV>
struct LocCfg {
    static constexpr int TB = NT / DK, L = C / TB;
    static constexpr int KT = DK / 16, VT = DV / 16;
    static constexpr int ES = (int)sizeof(In);
    static constexpr bool HL = ES == 2;       // bf16 inputs: split copies in the record
    static constexpr int LDF = DK + 4;        // fp32 [64][DK]
    static constexpr int LDT = DK + 16 / ES;  // In [64][DK]
    static constexpr int LDC = C + 4;         // fp32 [64][64]
    static constexpr int LDW = DV + 4;        // fp32 [64][DV]
    // operand tiles.  Pivoted chunk: KG = b.k.Gamma, KI = k / Gamma, QG = q.Gamma.  Other chunk,
    // while A and P are formed: G (fp32, block-local) and the raw k, b, q; afterwards KG.
    static constexpr int KG = 0, KI = C * LDF * 4, QG = 2 * C * LDF * 4;
    static constexpr int GG = 0, RK = C * LDF * 4, RB = RK + C * LDT * ES, RQ = RB + C * LDT * ES;
    static constexpr int TILES = cmax(3 * C * LDF * 4, RQ + C * LDT * ES);
    static constexpr int AT = TILES;               // [64][LDC] A, then T in place
    static constexpr int WV = AT + C * LDC * 4;    // [64][LDW] w.v
    static constexpr int TOT = WV + C * LDW * 4;   // [TB][DK] block sums of log alpha
    static constexpr int OFH = TOT + TB * DK * 4;  // [TB][DK] sums over the earlier blocks, hi
    static constexpr int OFL = OFH + TB * DK * 4;  // and lo
    static constexpr int FLG = OFL + TB * DK * 4;
    static constexpr int BYTES = FLG + 16;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(NT % DK == 0 && (KT + VT) % 4 == 0, "shape");
    static_assert(C * LDC * 4 <= QG - KI, "P does not fit over k / Gamma");
    static_assert(4 * 4 * 256 * 4 <= AT - QG, "the diagonal inverses' scratch does not fit");
    static_assert(8 * (KT + VT) / 2 * 256 * 4 <= AT, "the W and U0 staging does not fit");
};

template <typename In, int DK, int DV>
__global__ __launch_bounds__(NT) void bwd_local_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ bgate, const In* __restrict__ wgate,
    float* __restrict__ loc, int T, int H, int nper) {
    using G = LocCfg<In, DK, DV>;
    using R = Rec<DK, DV>;
    constexpr int TB = G::TB, L = G::L, KT = G::KT, VT = G::VT;
    constexpr int LDF = G::LDF, LDT = G::LDT, LDC = G::LDC, LDW = G::LDW;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    float* sKG = reinterpret_cast<float*>(smem + G::KG);
    float* sKI = reinterpret_cast<float*>(smem + G::KI);
    float* sQG = reinterpret_cast<float*>(smem + G::QG);
    float* sG = reinterpret_cast<float*>(smem + G::GG);
    In* sRK = reinterpret_cast<In*>(smem + G::RK);
    In* sRB = reinterpret_cast<In*>(smem + G::RB);
    In* sRQ = reinterpret_cast<In*>(smem + G::RQ);
    float* sWV = reinterpret_cast<float*>(smem + G::WV);
    float* sPS = reinterpret_cast<float*>(smem + G::KI);  // P, after A and P are formed
    float* sStage = reinterpret_cast<float*>(smem);       // the record's W and U0 tiles, per wave
    float* sAT = reinterpret_cast<float*>(smem + G::AT);
    float* sTOT = reinterpret_cast<float*>(smem + G::TOT);
    float* sOFH = reinterpret_cast<float*>(smem + G::OFH);
    float* sOFL = reinterpret_cast<float*>(smem + G::OFL);
    int* sFLG = reinterpret_cast<int*>(smem + G::FLG);

    const int tid_ = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid_ >> 6);
    const int lane_ = tid_ & 63, lane16 = lane_ & 15, grp4 = lane_ >> 4;
    const int nch = (T + C - 1) / C;
    const int ngrp = (nch + nper - 1) / nper;
    const int bh = blockIdx.x / ngrp, n0 = (blockIdx.x % ngrp) * nper, n1 = min(nch, n0 + nper);
    const int bi = bh / H, h = bh % H;
    const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;
    const int64_t base_k = ((int64_t)bi * T * H + h) * DK;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;

    const int ec_ = tid_ % DK;
    static_assert(DK % 64 == 0, "a wave's threads share one token block");
    constexpr int NWV = C * DV / 4 / NT;  // groups of 4 value columns per thread
    static_assert(NWV * 4 * NT == C * DV, "w.v split");
    KeyIn<In, L> in;
    Vec<In, 4> wr[NWV], vr[NWV];
    auto prefetch = [&](int nn) {
        const int tt0 = nn * C;
        load_key<In, L>(in, q, k, bgate, log_alpha, base_k, ec_, rk, tt0 + wave * 64 / DK * L, T);
#pragma unroll
        for (int i = 0; i < NWV; ++i) {
            const int e = tid_ + i * NT, r = e / (DV / 4), c4 = (e % (DV / 4)) * 4;
            const int64_t o = base_v + (int64_t)min(tt0 + r, T - 1) * rv + c4;
            wr[i] = load_vec<In, 4>(wgate + o);
            vr[i] = load_vec<In, 4>(v + o);
        }
    };
    if (n0 < n1) prefetch(n0);
    for (int n = n0; n < n1; ++n) {
        // lane indices opaque per chunk: loop-invariant values derived from them (masks, the
        // identity columns of the substitution) would otherwise stay live across the loop
        const int l16 = opq(lane16), g4 = opq(grp4), ec = opq(ec_);
        const int etb = wave * 64 / DK;  // = thread / DK: the threads of a wave share a token block
        const int tid = opq(tid_), lane = tid & 63;
        const int t0 = n * C;
        float* rec = loc + ((int64_t)bh * nch + n) * R::SIZE;
        if (tid == 0) *sFLG = 0;
        // element phase, pass 1: cumulative log-decay within the token block; w.v (exact in fp32)
        float x[L];
        {
            float run = 0.f;
#pragma unroll
            for (int m = 0; m < L; ++m) {
                run += t0 + etb * L + m < T ? in.g[m] : 0.f;
                x[m] = run;
            }
            sTOT[etb * DK + ec] = run;
#pragma unroll
            for (int i = 0; i < NWV; ++i) {
                const int e = tid + i * NT, r = e / (DV / 4), c4 = (e % (DV / 4)) * 4;
                f32x4 wv = zero4();
                if (t0 + r < T) {
#pragma unroll
                    for (int z = 0; z < 4; ++z) wv[z] = to_f32(wr[i].v[z]) * to_f32(vr[i].v[z]);
                }
                *reinterpret_cast<f32x4*>(sWV + r * LDW + c4) = wv;
            }
        }
        lds_barrier();
        float off = 0.f, after = 0.f;
        {
            float tot = 0.f, oh = 0.f, ol = 0.f;
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const float vj = sTOT[j * DK + ec];
                tot += vj;
                if (j < etb) {
                    off += vj;
                    float sv, ev;
                    two_sum(oh, vj, sv, ev);
                    oh = sv;
                    ol += ev;
                }
                if (j > etb) after += vj;
            }
            sOFH[etb * DK + ec] = oh;
            sOFL[etb * DK + ec] = ol;
            if (etb == 0) {
                rec[R::OGC + ec] = exp_any(tot);
                if (!(tot >= kMildLog)) *sFLG = 1;
            }
        }
        const float run = x[L - 1];
        lds_barrier();
        const bool mild = *sFLG == 0;
        // element phase, pass 2: QG and KR = k.Gamma_C / Gamma (suffix sums) to the record;
        // operand tiles of A and P
        float qgv[L], krv[L], gav[L];
        In qin[L], kin[L], bin[L];
        float* const krow = rec + R::OKR + etb * L * DK;  // this wave's first token row of KR
#pragma unroll
        for (int m = 0; m < L; ++m) {
            const int t = t0 + etb * L + m;
            qin[m] = kin[m] = bin[m] = from_f32<In>(0.f);
            if (t < T) {
                qin[m] = in.q[m];
                kin[m] = in.k[m];
                bin[m] = in.b[m];
            }
            gav[m] = exp_any(x[m] + off);
            qgv[m] = to_f32(qin[m]) * gav[m];
            krv[m] = to_f32(kin[m]) * exp_any((run - x[m]) + after);
            if constexpr (!G::HL) *at_byte(krow + m * DK, (uint32_t)ec * 4u) = krv[m];  // (bf16: split copy only)
        }
        if (mild) {
#pragma unroll
            for (int m = 0; m < L; ++m) {
                const int i = etb * L + m;
                sKG[i * LDF + ec] = to_f32(bin[m]) * to_f32(kin[m]) * gav[m];
                sKI[i * LDF + ec] = to_f32(kin[m]) * exp_any(-(x[m] + off));
                sQG[i * LDF + ec] = qgv[m];
            }
        } else {
#pragma unroll
            for (int m = 0; m < L; ++m) {
                const int i = etb * L + m;
                sG[i * LDF + ec] = x[m];  // block-local
                sRK[i * LDT + ec] = kin[m];
                sRB[i * LDT + ec] = bin[m];
                sRQ[i * LDT + ec] = qin[m];
            }
        }
        if constexpr (G::HL) {  // split copies: this thread's tokens, eight at a time
#pragma unroll
            for (int h8 = 0; h8 < L / 8; ++h8) {
                float a[8], b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a[e] = qgv[8 * h8 + e];
                    b[e] = krv[8 * h8 + e];
                }
                const int u = hl_unit(etb * L + 8 * h8, ec);
                put_hl8(reinterpret_cast<bf16*>(rec + R::OQG), C * DK, u, a);
                put_hl8(reinterpret_cast<bf16*>(rec + R::OKRS), C * DK, u, b);
            }
        } else {  // swizzled copies: this thread's tokens with one residue mod 4 are consecutive
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float a[L / 4], b[L / 4];
#pragma unroll
                for (int u = 0; u < L / 4; ++u) {
                    a[u] = qgv[g + 4 * u];
                    b[u] = krv[g + 4 * u];
                }
                store_n<L / 4>(rec + R::OQG + sw(etb * L + g, ec), a);
                store_n<L / 4>(rec + R::OKRS + sw(etb * L + g, ec), b);
            }
        }
        prefetch(min(n + 1, n1 - 1));  // on every path (see the serial kernels)
        lds_barrier();
        // A (strictly lower, into the A/T tile) and P (lower, to the record)
        if (mild) {
            // lower 16 x 16 blocks (I >= J) in the order (0,0) (1,0) (1,1) (2,0) ...: blocks 0-9 of
            // A, blocks 10-19 of P; wave w takes blocks w, w + 8, w + 16
            auto blk = [](int u, int& I, int& J) {
                const int x = u % 10;
                I = x < 1 ? 0 : (x < 3 ? 1 : (x < 6 ? 2 : 3));
                J = x - I * (I + 1) / 2;
            };
            f32x4 acc[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) acc[t] = zero4();
            mm_n<3, DK>(acc,
                [&](int t, int m, int kk) {
                    int I, J;
                    blk(wave + 8 * t, I, J);
                    return (wave + 8 * t >= 10 ? sQG : sKG)[(I * 16 + m) * LDF + kk];
                },
                [&](int t, int kk, int nn) {
                    int I, J;
                    blk(wave + 8 * t, I, J);
                    return sKI[(J * 16 + nn) * LDF + kk];
                }, l16, g4);
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int u = wave + 8 * t;
                if (u >= 10) continue;
                int I, J;
                blk(u, I, J);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = I * 16 + g4 * 4 + r, j = J * 16 + l16;
                    sAT[i * LDC + j] = j < i ? acc[t][r] : 0.f;
                }
            }
            lds_barrier();
            // P's lower blocks to their tile over k / Gamma (read by every wave until here)
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int u = wave + 8 * t;
                if (u < 10 || u >= 20) continue;
                int I, J;
                blk(u, I, J);
#pragma unroll
                for (int r = 0; r < 4; ++r) sPS[(I * 16 + g4 * 4 + r) * LDC + J * 16 + l16] = acc[t][r];
            }
        } else {
            const int i = tid & 63, jg = tid >> 6;
            const int bI = i / L;
            float pv[C / 8];
#pragma unroll
            for (int m = 0; m < C / 8; ++m) {
                const int j = jg + 8 * m;
                float a = 0.f, p = 0.f;
                if (j <= i) {
                    const int bJ = j / L;
                    for (int cc = 0; cc < DK; ++cc) {
                        const float dx = (sG[i * LDF + cc] - sG[j * LDF + cc]) +
                                         ((sOFH[bI * DK + cc] - sOFH[bJ * DK + cc]) +
                                          (sOFL[bI * DK + cc] - sOFL[bJ * DK + cc]));
                        const float f = exp_any(dx) * to_f32(sRK[j * LDT + cc]);
                        a += to_f32(sRB[i * LDT + cc]) * to_f32(sRK[i * LDT + cc]) * f;
                        p += to_f32(sRQ[i * LDT + cc]) * f;
                    }
                }
                sAT[i * LDC + j] = j < i ? a : 0.f;
                pv[m] = p;
            }
            lds_barrier();
#pragma unroll
            for (int m = 0; m < C / 8; ++m) sPS[i * LDC + jg + 8 * m] = pv[m];
        }
        // KG of the other kind of chunk (k and b reloaded: keeping the raw inputs live costs
        // registers everywhere), over the tiles A and P no longer need
        if (!mild) {
#pragma unroll
            for (int m = 0; m < L; ++m) {
                const int i = etb * L + m, t = t0 + i;
                float kv = 0.f, bv = 0.f;
                if (t < T) {
                    const int64_t o = base_k + (int64_t)t * rk + ec;
                    kv = to_f32(k[o]);
                    bv = to_f32(bgate[o]);
                }
                sKG[i * LDF + ec] = bv * kv * exp_any(x[m] + off);
            }
        }
        // T = (I + A)^{-1}: diagonal block I on wave I, in place.  N = A_II is strictly lower,
        // so N^16 = 0 and (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8): six 16 x 16 products
        // on fp32 MFMA through this wave's scratch over the QG tile (free once A and P exist)
        if (wave < 4) {
            float* mN = reinterpret_cast<float*>(smem + G::QG) + wave * 4 * 256;  // [16][16] each
            float* mN2 = mN + 256;
            float* mN4 = mN + 512;
            float* mM = mN + 768;
            float* mN8 = mN;  // N is last read for N^3
            float* Ab = sAT + wave * 16 * LDC + wave * 16;
            auto sync = [] {  // the wave's own LDS writes, before other lanes read them
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
            };
            auto put = [&](float* Z, const f32x4& x) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Z[(4 * g4 + r) * 16 + l16] = x[r];
            };
            auto prod = [&](const float* X, const float* Y) {  // X Y; lane holds rows 4 g4 + r of column l16
                f32x4 acc = zero4();
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) acc = mfma4(acc, X[l16 * 16 + 4 * g4 + s4], Y[(4 * g4 + s4) * 16 + l16]);
                return acc;
            };
            f32x4 n;
#pragma unroll
            for (int r = 0; r < 4; ++r) n[r] = Ab[(4 * g4 + r) * LDC + l16];
            put(mN, n);
            sync();
            const f32x4 n2 = prod(mN, mN);
            put(mN2, n2);
            sync();
            const f32x4 n4 = prod(mN2, mN2), n3 = prod(mN, mN2);
            put(mN4, n4);
            f32x4 m;  // (I - N)(I + N^2) = I - N + N^2 - N^3
#pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = (4 * g4 + r == l16 ? 1.f : 0.f) - n[r] + n2[r] - n3[r];
            put(mM, m);
            sync();
            const f32x4 n8 = prod(mN4, mN4);
            m += prod(mM, mN4);  // times (I + N^4)
            put(mN8, n8);
            sync();
            put(mM, m);  // after every lane's reads of the previous contents (one wave, in order)
            sync();
            m += prod(mM, mN8);  // times (I + N^8)
#pragma unroll
            for (int r = 0; r < 4; ++r) Ab[(4 * g4 + r) * LDC + l16] = m[r];
        }
        // off-diagonal blocks of T through halves of 32 tokens: T = [[T_A, 0], [T_C, T_B]] with
        // T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22 and the blocks of T_C from
        // Z_xJ = sum_{K=J}^{1} A_xK T_KJ: T_2J = -T_22 Z_2J, T_3J = -T_33 (Z_3J + A_32 T_2J).
        // Every wave first takes the rows of A it needs (T is formed in place over A; the
        // diagonal blocks above touch no off-diagonal block, so one barrier covers both); then wave
        // (R, J) = (2 + w / 2, w % 2), w < 4, forms its block of T_C with T_10 and T_2J in its own
        // registers, and waves 4 and 5 form and store T_10 and T_32: one step, no levels.
        // Operands: a row of a 16 x 16 block, lane (m, g4) holding X[m][4 g4 + e], times a block
        // that is a diagonal block of T in LDS or an accumulator (rows 4 g4 + r of column n).
        {
            auto arow = [&](int I, int J) {
                return *reinterpret_cast<const f32x4*>(sAT + (I * 16 + l16) * LDC + J * 16 + 4 * g4);
            };
            auto times_diag = [&](f32x4 acc, const f32x4& x, int D) {  // acc + X T_DD
    #pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(acc, x[e], sAT[(D * 16 + 4 * g4 + e) * LDC + D * 16 + l16]);
                return acc;
            };
            auto times_acc = [&](f32x4 acc, const f32x4& x, const f32x4& z) {  // acc + X Z
    #pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(acc, x[e], z[e]);
                return acc;
            };
            auto neg_diag_times = [&](int D, const f32x4& z) {  // -T_DD Z
                return -times_acc(zero4(), arow(D, D), z);
            };
            auto put = [&](int I, int J, const f32x4& t) {
    #pragma unroll
                for (int r = 0; r < 4; ++r) sAT[(I * 16 + g4 * 4 + r) * LDC + J * 16 + l16] = t[r];
            };
            const int J = wave & 1, R = 2 + ((wave >> 1) & 1);
            const bool tc = wave < 4, need10 = (tc && J == 0) || wave == 4;
            f32x4 a10 = zero4(), a2J = zero4(), a21 = zero4(), a3J = zero4(), a31 = zero4(), a32 = zero4();
            if (need10) a10 = arow(1, 0);
            if (tc) {
                a2J = arow(2, J);
                if (J == 0) a21 = arow(2, 1);
                if (R == 3) {
                    a3J = arow(3, J);
                    if (J == 0) a31 = arow(3, 1);
                }
            }
            if ((tc && R == 3) || wave == 5) a32 = arow(3, 2);
            lds_barrier();  // T's diagonal blocks complete, every row of A taken
            if (need10 || tc) {
                f32x4 t10 = zero4();
                if (need10) t10 = neg_diag_times(1, times_diag(zero4(), a10, 0));
                if (wave == 4) put(1, 0, t10);
                if (tc) {
                    f32x4 z2 = times_diag(zero4(), a2J, J);
                    if (J == 0) z2 = times_acc(z2, a21, t10);
                    const f32x4 t2 = neg_diag_times(2, z2);
                    if (R == 2) {
                        put(2, J, t2);
                    } else {
                        f32x4 z3 = times_diag(zero4(), a3J, J);
                        if (J == 0) z3 = times_acc(z3, a31, t10);
                        z3 = times_acc(z3, a32, t2);
                        put(3, J, neg_diag_times(3, z3));
                    }
                }
            } else if (wave == 5) {
                put(3, 2, neg_diag_times(3, times_diag(zero4(), a32, 2)));
            }
            lds_barrier();
        }
        // T and P to the record, swizzled, zero above the diagonal: 16-byte unit u holds rows
        // 16 j4 + 4 x + g (x = 0..3) of column 16 b + n16, u = ((4 b + j4) 4 + g) 16 + n16
#pragma unroll
        for (int y = 0; y < 2 * C * C / 4 / NT; ++y) {
            const int e = tid + y * NT, mat = e / (C * C / 4), u = e % (C * C / 4);
            if (G::HL && mat == 0) continue;  // T goes split (below)
            const int n16 = u & 15, g = (u >> 4) & 3, j4 = (u >> 6) & 3, b = u >> 8;
            const int c = 16 * b + n16;
            const float* src = mat ? sPS : sAT;
            f32x4 val;
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int i = 16 * j4 + 4 * z + g;
                val[z] = c <= i ? src[i * LDC + c] : 0.f;
            }
            *reinterpret_cast<f32x4*>(rec + (mat ? R::OP : R::OT) + 4 * u) = val;
        }
        if constexpr (G::HL) {  // T split: unit u holds rows 32 b2 + 8 g + e of column 16 cb + n16
            static_assert(C * C / 8 == NT, "one unit of T per thread");
            const int u = tid, n16 = u & 15, g = (u >> 4) & 3, b2 = (u >> 6) & 1, cb = u >> 7;
            const int c = 16 * cb + n16;
            float x[8];
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const int i = 32 * b2 + 8 * g + e2;
                x[e2] = c <= i ? sAT[i * LDC + c] : 0.f;
            }
            put_hl8(reinterpret_cast<bf16*>(rec + R::OT), C * C, u, x);
        }
        // W = T KG and U0 = T (w.v): wave w takes the row tiles p and 3 - p (p = w mod 2) of the
        // column tiles cg, cg + 4, ... (cg = w / 2) of [W | U0]; T is lower triangular, so row
        // tile I runs over the contraction blocks 0..I only
        {
            constexpr int NCOL = (KT + VT) / 4;
            const int p = wave & 1, cg = wave >> 1;
            f32x4 acc0[NCOL], acc1[NCOL];
#pragma unroll
            for (int c = 0; c < NCOL; ++c) acc0[c] = acc1[c] = zero4();
            // lane group g4 takes the tokens 16 kb + 4 g4 + s at step s: T's rows as 16-byte reads
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(sAT + (p * 16 + l16) * LDC + kb * 16 + 4 * g4);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(sAT + ((3 - p) * 16 + l16) * LDC + kb * 16 + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kk = kb * 16 + 4 * g4 + s;
                    float bc[NCOL];
#pragma unroll
                    for (int c = 0; c < NCOL; ++c) {
                        const int ct = cg + 4 * c;
                        bc[c] = ct < KT ? sKG[kk * LDF + ct * 16 + l16] : sWV[kk * LDW + (ct - KT) * 16 + l16];
                    }
#pragma unroll
                    for (int c = 0; c < NCOL; ++c) {
                        if (kb <= p) acc0[c] = mfma4(acc0[c], a0[s], bc[c]);
                        if (kb <= 3 - p) acc1[c] = mfma4(acc1[c], a1[s], bc[c]);
                    }
                }
            }
            // to the record in 16-byte rows, through a staging area of this wave's own (once
            // every wave is done with the operand tiles)
            lds_barrier();
            float* stg = sStage + wave * (2 * NCOL * 256);
#pragma unroll
            for (int c = 0; c < NCOL; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    stg[(2 * c) * 256 + (g4 * 4 + r) * 16 + l16] = acc0[c][r];
                    stg[(2 * c + 1) * 256 + (g4 * 4 + r) * 16 + l16] = acc1[c][r];
                }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own staging writes
            __builtin_amdgcn_wave_barrier();
            const int row = lane >> 2, q4 = (lane & 3) * 4;
#pragma unroll
            for (int c = 0; c < NCOL; ++c) {
                const int ct = cg + 4 * c;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int I = h2 ? 3 - p : p;
                    const float* tile = stg + (2 * c + h2) * 256;
                    const f32x4 val = *reinterpret_cast<const f32x4*>(tile + row * 16 + q4);
                    float* dst = ct < KT ? rec + R::OW + (I * 16 + row) * DK + ct * 16 + q4
                                         : rec + R::OU0 + (I * 16 + row) * DV + (ct - KT) * 16 + q4;
                    if (!G::HL || ct >= KT) *reinterpret_cast<f32x4*>(dst) = val;  // (bf16: W split only)
                    if constexpr (G::HL) {
                        if (ct < KT) {  // W split: lane (plane, half, column) writes rows 8 half + e
                            const int hf = (lane >> 4) & 1, pl = lane >> 5;
                            float x[8];
#pragma unroll
                            for (int e2 = 0; e2 < 8; ++e2) x[e2] = tile[(8 * hf + e2) * 16 + l16];
                            bf16x8 hi, lo;
                            split_hl8(x, hi, lo);
                            *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(rec + R::OWS) + pl * C * DK +
                                                       hl_unit(I * 16 + 8 * hf, ct * 16 + l16) * 8) = pl ? lo : hi;
                        }
                    } else if (ct < KT) {  // W swizzled: rows 4 x + g of column l16, as one unit
                        f32x4 sv4;
#pragma unroll
                        for (int x = 0; x < 4; ++x) sv4[x] = tile[(4 * x + g4) * 16 + l16];
                        *reinterpret_cast<f32x4*>(rec + R::OWS + sw(I * 16 + g4, ct * 16 + l16)) = sv4;
                    }
                }
            }
        }
        // the next chunk's first LDS writes (block sums, flag) touch nothing read above, and its
        // operand tiles come after two barriers
    }
}

// ---------------------------------------------------------------------------------------
// Kernels 1 and 2 walk the chunks of one (sequence, head, slice of value columns) in order.
// The slice's state (or state gradient) lives in MFMA accumulators as 16 x 16 tiles: wave w
// holds key rows 16 st .. 16 st + 15 (st = w mod KT) of SPW consecutive column tiles from
// cb = SPW (w / KT).  A product over the key axis with the state as right operand runs as
// eight partial products, one per wave over its own 16 rows (the accumulator layout is the
// operand layout), summed in LDS.  Two tiles per wave at dk = 128 (32-column slices): each
// record entry a wave loads serves both, and one workgroup per compute unit suffices.
// ---------------------------------------------------------------------------------------
template <int DK, int DV>
struct SerCfg {
    static constexpr int KT = DK / 16;
    static constexpr int SPW = KT == 8 ? 2 : 1;  // column tiles per wave
    static constexpr int NCT = 8 / KT * SPW;     // column tiles of a slice
    static constexpr int DVS = 16 * NCT;         // value columns of a slice
    static constexpr int NSL = DV / DVS;         // slices
    static constexpr int OPT = C * DVS / NT;     // summed outputs per thread (consecutive columns)
    static constexpr int TPR = DVS / OPT;        // threads per row of the sums
    static_assert(KT * NCT == 8 * SPW && DV % DVS == 0 && (OPT == 2 || OPT == 4), "shape");
};

// Kernel 1: the forward re-run, U = U0 - W S and S <- Gamma_C.S + KR^T U per chunk; stores
// the state entering every chunk and U
template <int DK, int DV, bool HL>
__global__ __launch_bounds__(NT) void bwd_fwd_kernel(const float* __restrict__ loc,
                                                     const float* __restrict__ initial_state,
                                                     float* __restrict__ s_ckpt, float* __restrict__ u_out,
                                                     int T, int H, int BH) {
    using SC = SerCfg<DK, DV>;
    using R = Rec<DK, DV>;
    constexpr int KT = SC::KT, SPW = SC::SPW, DVS = SC::DVS, OPT = SC::OPT, TPR = SC::TPR;
    __shared__ __attribute__((aligned(16))) float sPart[8 * SPW * C * 16];
    // U: fp32 [64][DVS], or (HL) transposed hi and lo bf16 planes [DVS][LDU]
    constexpr int LDU = C + 8;
    __shared__ __attribute__((aligned(16))) float sU[HL ? 4 : C * DVS];
    __shared__ __attribute__((aligned(16))) bf16 sUt[HL ? 2 * DVS * LDU : 8];
    // (HL) this wave's 16 columns of W (its key rows of the state) for all 64 tokens, hi and lo
    // planes [64][LWT], staged from the record's split copy (tokens contiguous) so that a lane
    // reads four consecutive keys of a token
    constexpr int LWT = 20;
    __shared__ __attribute__((aligned(16))) bf16 sWt[HL ? 8 * 2 * C * LWT : 8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    // the slices of one sequence and head are BH workgroups apart: on the same L2 when BH is a
    // multiple of the XCD count
    const int bh = blockIdx.x % BH, slice = blockIdx.x / BH;
    const int bi = bh / H, h = bh % H, col0 = slice * DVS;
    const int nch = (T + C - 1) / C;
    const int st = wave % KT, cb = (wave / KT) * SPW;
    const int64_t rv = (int64_t)H * DV;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;
    const int ri = tid / TPR, rc = (tid % TPR) * OPT;  // summed outputs: row ri, columns rc..
    const int rct = rc / 16, rcc = rc % 16;

    f32x4 S[SPW];
#pragma unroll
    for (int c = 0; c < SPW; ++c) {
        S[c] = zero4();
        if (initial_state) {
            const float* src = initial_state + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + (cb + c) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[c][r] = src[(int64_t)r * DV];
        }
    }
    // record entries are loaded one chunk ahead, each part right after its last use
    f32x4 Wv[4], GCv;
    bf16x8 Wu[2][2];  // (HL) split units of W: tokens 8 (g4 + 4 u) .. + 7 of key 16 st + l16
    float KRv[16], U0v[OPT];
    bf16x8 KRh[2], KRl[2];  // (HL) KR[32 b2 + 8 g4 + e][16 st + l16], split
    auto rec_of = [&](int nn) { return loc + ((int64_t)bh * nch + nn) * R::SIZE; };
    auto pre_w = [&](int nn) {
        const float* rec = rec_of(nn);
        if constexpr (HL) {  // the wave's units are contiguous: hl_unit(8 (g4 + 4 u), 16 st + l16)
            const bf16* wp = reinterpret_cast<const bf16*>(rec + R::OWS) + (st * 128 + lane) * 8;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl) Wu[u][pl] = *reinterpret_cast<const bf16x8*>(wp + u * 512 + pl * C * DK);
        } else {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                Wv[it] = *reinterpret_cast<const f32x4*>(rec + R::OW + (it * 16 + l16) * DK + st * 16 + g4 * 4);
        }
    };
    bf16* const wt = sWt + wave * 2 * C * LWT;
    auto stage_w = [&]() {  // (HL) the units to the wave's tile: token rows, key columns
        if constexpr (HL) {
            stage_key_pairs<LWT>(wt, Wu, l16, g4);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's writes before its reads
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
        }
    };
    auto pre_u0 = [&](int nn) { load_n<OPT>(U0v, rec_of(nn) + R::OU0 + ri * DV + col0 + rc); };
    auto pre_kr = [&](int nn) {
        const float* rec = rec_of(nn);
        if constexpr (HL) {
            const bf16* kp = reinterpret_cast<const bf16*>(rec + R::OKRS);
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int u = hl_unit(32 * b2 + 8 * g4, st * 16 + l16);
                KRh[b2] = *reinterpret_cast<const bf16x8*>(kp + u * 8);
                KRl[b2] = *reinterpret_cast<const bf16x8*>(kp + C * DK + u * 8);
            }
        } else {
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {  // KR[4 j + g4][16 st + l16], j = 0..15 (swizzled copy)
                const f32x4 x = *reinterpret_cast<const f32x4*>(rec + R::OKRS + sw(16 * j4 + g4, st * 16 + l16));
#pragma unroll
                for (int z = 0; z < 4; ++z) KRv[4 * j4 + z] = x[z];
            }
        }
        GCv = *reinterpret_cast<const f32x4*>(rec + R::OGC + st * 16 + g4 * 4);
    };
    pre_w(0);
    stage_w();
    pre_u0(0);
    pre_kr(0);
    // The prefetches are issued on every path (the last chunk loads its own record again): a
    // load skipped on some path makes the compiler's wait before each use cover every memory
    // operation still in flight.  A scheduling fence before each keeps the reload after the
    // last use, in the same registers.
    for (int n = 0; n < nch; ++n) {
        const int t0 = n * C, nn = min(n + 1, nch - 1);
        // checkpoint of the state entering the chunk
#pragma unroll
        for (int c = 0; c < SPW; ++c) {
            float* dst = s_ckpt + (((int64_t)bh * nch + n) * DK + st * 16 + g4 * 4) * DV + col0 + (cb + c) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)r * DV] = S[c][r];
        }
        // this wave's part of W S
        {
            f32x4 acc[SPW][4];
#pragma unroll
            for (int c = 0; c < SPW; ++c)
#pragma unroll
                for (int it = 0; it < 4; ++it) acc[c][it] = zero4();
            if constexpr (HL) {  // the accumulator rows 4 g4 + e are the K = 16 slots of the B operand
                bf16x4 sh[SPW], sl[SPW];
#pragma unroll
                for (int c = 0; c < SPW; ++c) split_hl(S[c], sh[c], sl[c]);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const bf16* wr = wt + (it * 16 + l16) * LWT + 4 * g4;
                    const bf16x4 wh = *reinterpret_cast<const bf16x4*>(wr);
                    const bf16x4 wl = *reinterpret_cast<const bf16x4*>(wr + C * LWT);
#pragma unroll
                    for (int c = 0; c < SPW; ++c)
                        acc[c][it] = mf16(mf16(mf16(acc[c][it], wh, sh[c]), wh, sl[c]), wl, sh[c]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int c = 0; c < SPW; ++c)
#pragma unroll
                        for (int it = 0; it < 4; ++it) acc[c][it] = mfma4(acc[c][it], Wv[it][j], S[c][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
            pre_w(nn);
#pragma unroll
            for (int c = 0; c < SPW; ++c)
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sPart[((wave * SPW + c) * C + it * 16 + g4 * 4 + r) * 16 + l16] = acc[c][it][r];
        }
        lds_barrier();
        // U = U0 - W S: the parts of column tile rct sit with the waves st' + KT (rct / SPW)
        {
            float u[OPT];
#pragma unroll
            for (int o = 0; o < OPT; ++o) u[o] = U0v[o];
#pragma unroll
            for (int s2 = 0; s2 < KT; ++s2) {
                const int w2 = s2 + KT * (rct / SPW);
                float p[OPT];
                load_n<OPT>(p, sPart + ((w2 * SPW + rct % SPW) * C + ri) * 16 + rcc);
#pragma unroll
                for (int o = 0; o < OPT; ++o) u[o] -= p[o];
            }
            if constexpr (HL) {
#pragma unroll
                for (int o = 0; o < OPT; ++o) {
                    const bf16 h = (bf16)u[o];
                    sUt[(rc + o) * LDU + ri] = h;
                    sUt[DVS * LDU + (rc + o) * LDU + ri] = (bf16)(u[o] - (float)h);
                }
            } else {
                store_n<OPT>(sU + ri * DVS + rc, u);
            }
            if (t0 + ri < T) store_n<OPT>(u_out + base_v + (int64_t)(t0 + ri) * rv + col0 + rc, u);
        }
        __builtin_amdgcn_sched_barrier(0);
        pre_u0(nn);
        lds_barrier();
        // S <- Gamma_C.S + KR^T U
        {
            f32x4 a2[SPW][2];
#pragma unroll
            for (int c = 0; c < SPW; ++c) {
#pragma unroll
                for (int r = 0; r < 4; ++r) a2[c][0][r] = S[c][r] * GCv[r];
                a2[c][1] = zero4();
            }
            if constexpr (HL) {  // slot (g4, e) of block b2: token 32 b2 + 8 g4 + e, split operands
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
                    for (int c = 0; c < SPW; ++c) {
                        const bf16* up = sUt + ((cb + c) * 16 + l16) * LDU + 32 * b2 + 8 * g4;
                        const bf16x8 uh = *reinterpret_cast<const bf16x8*>(up);
                        const bf16x8 ul = *reinterpret_cast<const bf16x8*>(up + DVS * LDU);
                        a2[c][b2] = mf32(mf32(mf32(a2[c][b2], KRh[b2], uh), KRh[b2], ul), KRl[b2], uh);
                    }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
#pragma unroll
                    for (int c = 0; c < SPW; ++c)
                        a2[c][j & 1] = mfma4(a2[c][j & 1], KRv[j], sU[(4 * j + g4) * DVS + (cb + c) * 16 + l16]);
            }
#pragma unroll
            for (int c = 0; c < SPW; ++c) {
                S[c] = a2[c][0] + a2[c][1];
                pin(S[c]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        pre_kr(nn);
        stage_w();  // the next chunk's W, loaded after this chunk's W S
    }
}

// Kernel 2: the chunks in reverse order, dU = P^T dO + KR dS', dS = Gamma_C.dS' + QG^T dO -
// W^T dU (W^T = KG^T T^T), dR = T^T dU; stores dS' of every chunk, dR, and the gradient of the
// initial state
template <int DK, int DV, bool HL>
__global__ __launch_bounds__(NT) void bwd_state_kernel(const float* __restrict__ loc, const float* __restrict__ d_o,
                                                       const float* __restrict__ d_final,
                                                       float* __restrict__ ds_ckpt, float* __restrict__ dr_out,
                                                       float* __restrict__ d_initial, int T, int H, int BH) {
    using SC = SerCfg<DK, DV>;
    using R = Rec<DK, DV>;
    constexpr int KT = SC::KT, SPW = SC::SPW, DVS = SC::DVS, OPT = SC::OPT, TPR = SC::TPR;
    constexpr int JW = C / KT;  // tokens of P^T dO in this wave's part
    constexpr int JS = JW / 4;  // their MFMA steps
    __shared__ __attribute__((aligned(16))) float sPart[8 * SPW * C * 16];
    // dU and dO: fp32 [64][DVS], or (HL) transposed hi and lo bf16 planes [DVS][LDU]
    constexpr int LDU = C + 8;
    __shared__ __attribute__((aligned(16))) float sDU[HL ? 4 : C * DVS];
    __shared__ __attribute__((aligned(16))) float sDO[2][HL ? 4 : C * DVS];
    __shared__ __attribute__((aligned(16))) bf16 sDUt[HL ? 2 * DVS * LDU : 8];
    __shared__ __attribute__((aligned(16))) bf16 sDOt[2][HL ? 2 * DVS * LDU : 8];
    // (HL) this wave's 16 columns of KR (its key rows of dS') for all 64 tokens, hi and lo planes
    // [64][LKT], staged from the record's split copy (tokens contiguous) so that a lane reads four
    // consecutive keys of a token
    constexpr int LKT = 20;
    __shared__ __attribute__((aligned(16))) bf16 sKt[HL ? 8 * 2 * C * LKT : 8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int bh = blockIdx.x % BH, slice = blockIdx.x / BH;
    const int bi = bh / H, h = bh % H, col0 = slice * DVS;
    const int nch = (T + C - 1) / C;
    const int st = wave % KT, cb = (wave / KT) * SPW;
    const int64_t rv = (int64_t)H * DV;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;
    const int ri = tid / TPR, rc = (tid % TPR) * OPT;
    const int rct = rc / 16, rcc = rc % 16;
    // dR tiles of this wave: row tile dri (waves with st < 4), its column tiles
    const bool has_dr = st < 4;
    const int dri = st & 3;

    f32x4 dS[SPW];
#pragma unroll
    for (int c = 0; c < SPW; ++c) {
        dS[c] = zero4();
        if (d_final) {
            const float* src = d_final + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + (cb + c) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[c][r] = src[(int64_t)r * DV];
        }
    }
    f32x4 KRv[4], GCv;
    bf16x8 Ku[2][2];  // (HL) split units of KR: tokens 8 (g4 + 4 u) .. + 7 of key 16 st + l16
    float Pv[4][JS], dOp[SPW][JS], dOs[OPT], QGv[16], Wt[16], Tv[16];
    bf16x8 QGh[2], QGl[2], Wh[2], Wl[2], Th[2], Tl[2];  // (HL) split, tokens 32 b2 + 8 g4 + e
    auto rec_of = [&](int nn) { return loc + ((int64_t)bh * nch + nn) * R::SIZE; };
    auto do_row = [&](int t) { return d_o + base_v + (int64_t)min(t, T - 1) * rv + col0; };
    auto pre_du = [&](int nn) {  // operands of the dU parts
        const float* rec = rec_of(nn);
        if constexpr (HL) {  // the wave's units are contiguous: hl_unit(8 (g4 + 4 u), 16 st + l16)
            const bf16* kp = reinterpret_cast<const bf16*>(rec + R::OKRS) + (st * 128 + lane) * 8;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl) Ku[u][pl] = *reinterpret_cast<const bf16x8*>(kp + u * 512 + pl * C * DK);
        } else {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                KRv[it] = *reinterpret_cast<const f32x4*>(rec + R::OKR + (it * 16 + l16) * DK + st * 16 + g4 * 4);
        }
        // P[st JW + 4 s + g4][16 it + l16], s = 0..JS-1: consecutive in the swizzled copy
#pragma unroll
        for (int it = 0; it < 4; ++it) load_n<JS>(Pv[it], rec + R::OP + sw(st * JW + g4, it * 16 + l16));
#pragma unroll
        for (int s = 0; s < JS; ++s) {
            const int j = st * JW + 4 * s + g4;
#pragma unroll
            for (int c = 0; c < SPW; ++c)
                dOp[c][s] = nn * C + j < T ? do_row(nn * C + j)[(cb + c) * 16 + l16] : 0.f;
        }
    };
    auto pre_do = [&](int nn) {  // the dO slice for LDS
        load_n<OPT>(dOs, do_row(nn * C + ri) + rc);
        if (nn * C + ri >= T) {
#pragma unroll
            for (int o = 0; o < OPT; ++o) dOs[o] = 0.f;
        }
    };
    auto pre_ds = [&](int nn) {  // operands of the dS update
        const float* rec = rec_of(nn);
        if constexpr (HL) {
            const bf16* qp = reinterpret_cast<const bf16*>(rec + R::OQG);
            const bf16* wp = reinterpret_cast<const bf16*>(rec + R::OWS);
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int u = hl_unit(32 * b2 + 8 * g4, st * 16 + l16);
                QGh[b2] = *reinterpret_cast<const bf16x8*>(qp + u * 8);
                QGl[b2] = *reinterpret_cast<const bf16x8*>(qp + C * DK + u * 8);
                Wh[b2] = *reinterpret_cast<const bf16x8*>(wp + u * 8);
                Wl[b2] = *reinterpret_cast<const bf16x8*>(wp + C * DK + u * 8);
            }
        } else
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {  // QG and W at [4 j + g4][16 st + l16] (swizzled copies)
            const f32x4 a = *reinterpret_cast<const f32x4*>(rec + R::OQG + sw(16 * j4 + g4, st * 16 + l16));
            const f32x4 b = *reinterpret_cast<const f32x4*>(rec + R::OWS + sw(16 * j4 + g4, st * 16 + l16));
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                QGv[4 * j4 + z] = a[z];
                Wt[4 * j4 + z] = b[z];
            }
        }
        GCv = *reinterpret_cast<const f32x4*>(rec + R::OGC + st * 16 + g4 * 4);
    };
    auto pre_t = [&](int nn) {  // T^T operand of the dR tile: T[j][16 dri + m], j >= 16 dri
        const float* rec = rec_of(nn);
        if (HL && has_dr) {  // T[32 b2 + 8 g4 + e][16 dri + l16], split
            const bf16* tp = reinterpret_cast<const bf16*>(rec + R::OT);
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int u = hl_unit(32 * b2 + 8 * g4, dri * 16 + l16);
                Th[b2] = *reinterpret_cast<const bf16x8*>(tp + u * 8);
                Tl[b2] = *reinterpret_cast<const bf16x8*>(tp + C * C + u * 8);
            }
        } else if (has_dr) {  // T[16 kb + 4 s + g4][16 dri + l16] (zero for kb < dri), swizzled copy
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(rec + R::OT + sw(16 * kb + g4, dri * 16 + l16));
#pragma unroll
                for (int z = 0; z < 4; ++z) Tv[kb * 4 + z] = x[z];
            }
        }
    };
    bf16* const kt = sKt + wave * 2 * C * LKT;
    auto stage_kr = [&]() {  // (HL) the units to the wave's tile: token rows, key columns
        if constexpr (HL) {
            stage_key_pairs<LKT>(kt, Ku, l16, g4);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's writes before its reads
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
        }
    };
    pre_du(nch - 1);
    stage_kr();
    pre_do(nch - 1);
    pre_ds(nch - 1);
    pre_t(nch - 1);
    // The prefetches are issued on every path (chunk 0 loads its own record again), each after
    // a scheduling fence that keeps it behind the last use (see kernel 1).
    for (int n = nch - 1; n >= 0; --n) {
        const int t0 = n * C, nn = max(n - 1, 0);
        float* sDOn = sDO[n & 1];
        bf16* sDOtn = sDOt[n & 1];
        // dS' of this chunk, checkpoint for kernel 3
#pragma unroll
        for (int c = 0; c < SPW; ++c) {
            float* dst = ds_ckpt + (((int64_t)bh * nch + n) * DK + st * 16 + g4 * 4) * DV + col0 + (cb + c) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)r * DV] = dS[c][r];
        }
        if constexpr (HL) {
#pragma unroll
            for (int o = 0; o < OPT; ++o) {
                const bf16 h = (bf16)dOs[o];
                sDOtn[(rc + o) * LDU + ri] = h;
                sDOtn[DVS * LDU + (rc + o) * LDU + ri] = (bf16)(dOs[o] - (float)h);
            }
        } else {
            store_n<OPT>(sDOn + ri * DVS + rc, dOs);
        }
        __builtin_amdgcn_sched_barrier(0);
        pre_do(nn);
        // this wave's parts of KR dS' (its 16 key rows) and of P^T dO (its JW tokens)
        {
            f32x4 acc[SPW][4];
#pragma unroll
            for (int c = 0; c < SPW; ++c)
#pragma unroll
                for (int it = 0; it < 4; ++it) acc[c][it] = zero4();
            if constexpr (HL) {  // the accumulator rows 4 g4 + e are the K = 16 slots of the B operand
                bf16x4 sh[SPW], sl[SPW];
#pragma unroll
                for (int c = 0; c < SPW; ++c) split_hl(dS[c], sh[c], sl[c]);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const bf16* kr = kt + (it * 16 + l16) * LKT + 4 * g4;
                    const bf16x4 kh = *reinterpret_cast<const bf16x4*>(kr);
                    const bf16x4 kl = *reinterpret_cast<const bf16x4*>(kr + C * LKT);
#pragma unroll
                    for (int c = 0; c < SPW; ++c)
                        acc[c][it] = mf16(mf16(mf16(acc[c][it], kh, sh[c]), kh, sl[c]), kl, sh[c]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int c = 0; c < SPW; ++c)
#pragma unroll
                        for (int it = 0; it < 4; ++it) acc[c][it] = mfma4(acc[c][it], KRv[it][j], dS[c][j]);
            }
#pragma unroll
            for (int s = 0; s < JS; ++s) {
                const int jb = (st * JW + 4 * s) / 16;  // token block: P[j][i] = 0 for row tiles past it
#pragma unroll
                for (int c = 0; c < SPW; ++c)
#pragma unroll
                    for (int it = 0; it < 4; ++it)
                        if (it <= jb) acc[c][it] = mfma4(acc[c][it], Pv[it][s], dOp[c][s]);
            }
            __builtin_amdgcn_sched_barrier(0);
            pre_du(nn);
#pragma unroll
            for (int c = 0; c < SPW; ++c)
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sPart[((wave * SPW + c) * C + it * 16 + g4 * 4 + r) * 16 + l16] = acc[c][it][r];
        }
        lds_barrier();
        // dU = sum of the parts of column tile rct
        {
            float u[OPT];
#pragma unroll
            for (int o = 0; o < OPT; ++o) u[o] = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < KT; ++s2) {
                const int w2 = s2 + KT * (rct / SPW);
                float p[OPT];
                load_n<OPT>(p, sPart + ((w2 * SPW + rct % SPW) * C + ri) * 16 + rcc);
#pragma unroll
                for (int o = 0; o < OPT; ++o) u[o] += p[o];
            }
            if constexpr (HL) {
#pragma unroll
                for (int o = 0; o < OPT; ++o) {
                    const bf16 h = (bf16)u[o];
                    sDUt[(rc + o) * LDU + ri] = h;
                    sDUt[DVS * LDU + (rc + o) * LDU + ri] = (bf16)(u[o] - (float)h);
                }
            } else {
                store_n<OPT>(sDU + ri * DVS + rc, u);
            }
        }
        lds_barrier();
        // dS <- Gamma_C.dS' + QG^T dO - W^T dU
        {
            f32x4 a2[SPW][2];
#pragma unroll
            for (int c = 0; c < SPW; ++c) a2[c][0] = a2[c][1] = zero4();
            if constexpr (HL) {  // slot (g4, e) of block b2: token 32 b2 + 8 g4 + e, split operands
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
                    for (int c = 0; c < SPW; ++c) {
                        const int o = ((cb + c) * 16 + l16) * LDU + 32 * b2 + 8 * g4;
                        const bf16x8 oh = *reinterpret_cast<const bf16x8*>(sDOtn + o);
                        const bf16x8 ol = *reinterpret_cast<const bf16x8*>(sDOtn + DVS * LDU + o);
                        const bf16x8 uh = *reinterpret_cast<const bf16x8*>(sDUt + o);
                        const bf16x8 ul = *reinterpret_cast<const bf16x8*>(sDUt + DVS * LDU + o);
                        a2[c][0] = mf32(mf32(mf32(a2[c][0], QGh[b2], oh), QGh[b2], ol), QGl[b2], oh);
                        a2[c][1] = mf32(mf32(mf32(a2[c][1], Wh[b2], uh), Wh[b2], ul), Wl[b2], uh);
                    }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
#pragma unroll
                    for (int c = 0; c < SPW; ++c) {
                        const int o = (4 * j + g4) * DVS + (cb + c) * 16 + l16;
                        a2[c][0] = mfma4(a2[c][0], QGv[j], sDOn[o]);
                        a2[c][1] = mfma4(a2[c][1], Wt[j], sDU[o]);
                    }
            }
#pragma unroll
            for (int c = 0; c < SPW; ++c) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dS[c][r] = dS[c][r] * GCv[r] + a2[c][0][r] - a2[c][1][r];
                pin(dS[c]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        pre_ds(nn);
        // dR = T^T dU (row tile dri)
        if (has_dr) {
            f32x4 acc[SPW][2];
#pragma unroll
            for (int c = 0; c < SPW; ++c) acc[c][0] = acc[c][1] = zero4();
            if constexpr (HL) {  // slot (g4, e) of block b2: token 32 b2 + 8 g4 + e; T is zero above
                                 // the diagonal, so block 0 adds nothing for row tiles 2 and 3
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2)
                    if (b2 == 1 || dri < 2) {
#pragma unroll
                        for (int c = 0; c < SPW; ++c) {
                            const int o = ((cb + c) * 16 + l16) * LDU + 32 * b2 + 8 * g4;
                            const bf16x8 uh = *reinterpret_cast<const bf16x8*>(sDUt + o);
                            const bf16x8 ul = *reinterpret_cast<const bf16x8*>(sDUt + DVS * LDU + o);
                            acc[c][b2] = mf32(mf32(mf32(acc[c][b2], Th[b2], uh), Th[b2], ul), Tl[b2], uh);
                        }
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    if (kb >= dri) {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
#pragma unroll
                            for (int c = 0; c < SPW; ++c)
                                acc[c][s & 1] = mfma4(acc[c][s & 1], Tv[kb * 4 + s],
                                                      sDU[(kb * 16 + 4 * s + g4) * DVS + (cb + c) * 16 + l16]);
                    }
            }
#pragma unroll
            for (int c = 0; c < SPW; ++c) {
                const f32x4 dr = acc[c][0] + acc[c][1];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = dri * 16 + g4 * 4 + r, t = t0 + i;
                    if (t < T) dr_out[base_v + (int64_t)t * rv + col0 + (cb + c) * 16 + l16] = dr[r];
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        pre_t(nn);
        stage_kr();  // the next chunk's KR, loaded after this chunk's partial products
    }
    if (d_initial) {
#pragma unroll
        for (int c = 0; c < SPW; ++c) {
            float* dst = d_initial + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + (cb + c) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)r * DV] = dS[c][r];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Kernel 3: all input gradients of one chunk
// ---------------------------------------------------------------------------------------
template <typename In, int DK, int DV>
struct GradCfg {
    static constexpr int TB = NT / DK, L = C / TB;
    static constexpr int KT = DK / 16;
    static constexpr int TPW = 4 * KT / 8;    // output tiles (token rows x channel columns) per wave
    static constexpr int ITS = 8 / KT;        // row-tile stride between a wave's tiles
    static constexpr int ES = (int)sizeof(In);
    static constexpr int LDV = DV + 4;        // fp32 [64][DV]
    static constexpr int LDH = DV / 2 + 4;    // fp32 [DK][DV/2]: half of S or dS'
    static constexpr int LDC = C + 4;         // fp32 [64][64]
    static constexpr int LDF = DK + 4;        // fp32 [64][DK]
    static constexpr int LDT = DK + 16 / ES;  // In [64][DK]
    // bf16 inputs: the phase 2-3 products on bf16 hi/lo operands, each matrix as a hi and a lo
    // plane of bf16 rows (LDB, LDS2 elements); fp32 inputs: fp32 rows
    static constexpr bool HL = ES == 2;
    static constexpr int LDB = DV + 8, LDS2 = DV / 2 + 8;
    static constexpr int PB = C * LDB * 2, PS = DK * LDS2 * 2;  // plane bytes
    static constexpr int MAT = HL ? 2 * PB : C * LDV * 4;       // dO, dR or U
    // region 1: dO, dR, U (phases 1-3); then G and the raw q, k, b (phases 3-5)
    static constexpr int DO = 0, DR = MAT, UU = 2 * MAT;
    static constexpr int GG = 0, QQ = C * LDF * 4, KK = QQ + C * LDT * ES, BB = KK + C * LDT * ES;
    static constexpr int R1 = cmax(3 * MAT, BB + C * LDT * ES);
    // region 2: a half of S or dS' (phase 2); then dA, dP (phases 3-4: fp32 tiles, or with bf16
    // inputs the packed planes below); then dG (phase 5, when a wave does not hold every token of
    // its channels)
    static constexpr int SH = R1, DA = R1, DP = R1 + C * LDC * 4, DG = R1;
    // bf16 inputs, phases 3-4: dA and dP as two packed matrices of hi and lo planes [64][LDM],
    // M1 = dP on and below the diagonal with dA^T above it, M2 = dA below with dP^T on and above
    static constexpr int LDM = C + 8, PM = C * LDM * 2;
    static constexpr int M1H = R1, M1L = R1 + PM, M2H = R1 + 2 * PM, M2L = R1 + 3 * PM;
    static constexpr int R2 = cmax(HL ? cmax(2 * PS, 4 * PM) : cmax(DK * LDH * 4, 2 * C * LDC * 4), C * LDF * 4);
    static constexpr int GC = R1 + R2;        // [DK] Gamma_C
    static constexpr int XD = GC + DK * 4;    // [DK] sum_v dS'[c][v] S[c][v]
    static constexpr int XR = XD + DK * 4;    // [DK] sum_i KR_ic (U dS'^T)_ic
    static constexpr int TOT = XR + DK * 4;   // [TB][DK] block sums of log alpha
    static constexpr int OFH = TOT + TB * DK * 4;  // [TB][DK] sums over the earlier blocks, hi
    static constexpr int OFL = OFH + TB * DK * 4;  // and lo
    static constexpr int AFT = OFL + TB * DK * 4;  // [TB][DK] sums over the later blocks
    static constexpr int FLG = AFT + TB * DK * 4;
    static constexpr int BYTES = FLG + 16;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(KT == 4 || KT == 8, "shape");
};

template <typename In, int DK, int DV>
__global__ __launch_bounds__(NT) void bwd_chunk_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ bgate, const In* __restrict__ wgate,
    const float* __restrict__ d_o, const float* __restrict__ s_ckpt, const float* __restrict__ ds_ckpt,
    const float* __restrict__ u_in, const float* __restrict__ dr_in, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg, float* __restrict__ db,
    float* __restrict__ dw, int T, int H, int nper) {
    using G = GradCfg<In, DK, DV>;
    constexpr int TB = G::TB, L = G::L, KT = G::KT, TPW = G::TPW, ITS = G::ITS;
    constexpr int LDV = G::LDV, LDH = G::LDH, LDC = G::LDC, LDF = G::LDF, LDT = G::LDT;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    float* sDO = reinterpret_cast<float*>(smem + G::DO);
    float* sDR = reinterpret_cast<float*>(smem + G::DR);
    float* sU = reinterpret_cast<float*>(smem + G::UU);
    float* sG = reinterpret_cast<float*>(smem + G::GG);
    In* sQ = reinterpret_cast<In*>(smem + G::QQ);
    In* sK = reinterpret_cast<In*>(smem + G::KK);
    In* sB = reinterpret_cast<In*>(smem + G::BB);
    float* sSH = reinterpret_cast<float*>(smem + G::SH);
    float* sDA = reinterpret_cast<float*>(smem + G::DA);
    float* sDP = reinterpret_cast<float*>(smem + G::DP);
    float* sDG = reinterpret_cast<float*>(smem + G::DG);
    float* sGC = reinterpret_cast<float*>(smem + G::GC);
    float* sXD = reinterpret_cast<float*>(smem + G::XD);
    float* sXR = reinterpret_cast<float*>(smem + G::XR);
    float* sTOT = reinterpret_cast<float*>(smem + G::TOT);
    float* sOFH = reinterpret_cast<float*>(smem + G::OFH);
    float* sOFL = reinterpret_cast<float*>(smem + G::OFL);
    float* sAFT = reinterpret_cast<float*>(smem + G::AFT);
    int* sFLG = reinterpret_cast<int*>(smem + G::FLG);
    constexpr int LDB = G::LDB, LDS2 = G::LDS2;
    // bf16 inputs: a matrix in LDS as hi and lo planes (npl elements apart)
    auto put_hl = [&](int off, int npl, int ld, int r, int c4, const f32x4& x) {
        bf16* hi = reinterpret_cast<bf16*>(smem + off) + r * ld + c4;
        bf16x4 h, l;
        split_hl(x, h, l);
        *reinterpret_cast<bf16x4*>(hi) = h;
        *reinterpret_cast<bf16x4*>(hi + npl) = l;
    };
    auto pl_of = [&](int off, int npl, int pl) { return reinterpret_cast<const bf16*>(smem + off) + pl * npl; };
    // entry (a, b) of a packed matrix (bf16 inputs, phases 3-4) as hi + lo
    auto pk = [&](int off, int a, int b) {
        const bf16* x = reinterpret_cast<const bf16*>(smem + off) + a * G::LDM + b;
        return (float)x[0] + (float)x[G::PM / 2];
    };
    // G_i (chunk-local), G_i - G_j and G_C - G_i from the block-local tile (see two_sum)
    auto Gof = [&](int i, int c) {
        const int b = i / L;
        return sG[i * LDF + c] + (sOFH[b * DK + c] + sOFL[b * DK + c]);
    };
    auto Gdiff = [&](int i, int j, int c) {
        const int bI = i / L, bJ = j / L;
        return (sG[i * LDF + c] - sG[j * LDF + c]) +
               ((sOFH[bI * DK + c] - sOFH[bJ * DK + c]) + (sOFL[bI * DK + c] - sOFL[bJ * DK + c]));
    };
    auto Gsuf = [&](int i, int c) {
        const int b = i / L;
        return (sTOT[b * DK + c] - sG[i * LDF + c]) + sAFT[b * DK + c];
    };

    const int tid_ = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid_ >> 6);
    // a run of nper consecutive chunks of one (sequence, head) per workgroup
    const int nch = (T + C - 1) / C;
    const int ngrp = (nch + nper - 1) / nper;
    const int bh = blockIdx.x / ngrp, n0 = (blockIdx.x % ngrp) * nper, n1 = min(nch, n0 + nper);
    const int bi = bh / H, h = bh % H;
    const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;
    const int64_t base_k = ((int64_t)bi * T * H + h) * DK;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;
    auto state_of = [&](const float* base, int nn) { return base + ((int64_t)bh * nch + nn) * DK * DV; };

    // this wave's output tiles: channel column tile ct, token row tiles it0 + ITS j
    const int ct = wave % KT, it0 = wave / KT;

    constexpr int HV = DV / 2;
    constexpr int NSH = DK * HV / 4 / NT;  // float4 of a half of S (or dS') per thread
    static_assert(NSH * 4 * NT == DK * HV, "half split");
    f32x4 sv[NSH], dsv[NSH];
    float xd[NSH];  // this thread's part of sum_v dS'[r][v] S[r][v] for its rows
    // (a wave-uniform row base plus a 32-bit lane offset for every global access below)
    auto load_half = [&](int lane, f32x4 (&d)[NSH], const float* g, int hh) {
#pragma unroll
        for (int i = 0; i < NSH; ++i) {
            const int rb = (wave * 64 + i * NT) / (HV / 4);
            const uint32_t lo = ((lane / (HV / 4)) * DV + (lane % (HV / 4)) * 4) * 4;
            d[i] = *reinterpret_cast<const f32x4*>(at_byte(g + rb * DV + hh * HV, lo));
        }
    };

    // ---- phase 1, by halves of the value axis: dO, dR, U of the chunk into LDS; dv = dR.w,
    // dw = dR.v.  The second half's loads are in flight during the first half's products ----
    constexpr int NP1 = C * HV / 4 / NT;  // float4 of a value half per thread
    static_assert(NP1 * 4 * NT == C * HV, "phase 1 split");
    f32x4 p1o[NP1], p1r[NP1], p1u[NP1];
    Vec<In, 4> p1w[NP1], p1v[NP1];
    auto p1_load = [&](int lane, int nn, int hh) {  // rows past the end read the last token, zeroed in p1_use
#pragma unroll
        for (int x = 0; x < NP1; ++x) {
            const int r0 = nn * C + (wave * 64 + x * NT) / (HV / 4);  // the wave's first row
            const int u = min(r0, T - 1);
            const int dl = min(r0 + lane / (HV / 4), T - 1) - u;      // the lane's row, from u
            const int c4 = hh * HV + (lane % (HV / 4)) * 4;
            const int64_t ro = base_v + (int64_t)u * rv;
            const uint32_t lo = (uint32_t)dl * (uint32_t)rv + (uint32_t)c4;
            p1o[x] = *reinterpret_cast<const f32x4*>(at_byte(d_o + ro, lo * 4));
            p1r[x] = *reinterpret_cast<const f32x4*>(at_byte(dr_in + ro, lo * 4));
            p1u[x] = *reinterpret_cast<const f32x4*>(at_byte(u_in + ro, lo * 4));
            p1w[x] = load_vec<In, 4>(at_byte(wgate + ro, lo * (uint32_t)sizeof(In)));
            p1v[x] = load_vec<In, 4>(at_byte(v + ro, lo * (uint32_t)sizeof(In)));
        }
    };
    // the first chunk's loads, in the order of use (a wait covers every load issued before the
    // one it needs); every later chunk's come during phase 5 of the chunk before it
    p1_load(tid_ & 63, n0, 0);
    load_half(tid_ & 63, sv, state_of(s_ckpt, n0), 0);
    load_half(tid_ & 63, dsv, state_of(ds_ckpt, n0), 0);
    // one chunk; FULL: every token of the chunk is in the sequence, so no store is conditional
    // (a conditional store would make the waits for the next chunk's loads, issued before it,
    // drain the stores that follow them)
    auto chunk = [&](const int n, auto full_c) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        // lane indices opaque per chunk: values derived from them (LDS addresses of the
        // products) would otherwise be hoisted out of the loop and stay live across it
        const int tid = opq(tid_);
        const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
        const int c = ct * 16 + l16;  // the channel of this lane's accumulator column
        auto p1_use = [&](int t0, int hh) {
    #pragma unroll
            for (int x = 0; x < NP1; ++x) {
                const int e = tid + x * NT, r = e / (HV / 4), c4 = hh * HV + (e % (HV / 4)) * 4, t = t0 + r;
                f32x4 o4 = zero4(), r4 = zero4(), u4 = zero4();
                if (FULL || t < T) {
                    o4 = p1o[x];
                    r4 = p1r[x];
                    u4 = p1u[x];
                    // a wave-uniform row base plus a 32-bit lane offset
                    const int64_t ro = base_v + (int64_t)(t0 + (wave * 64 + x * NT) / (HV / 4)) * rv;
                    const uint32_t lo = ((uint32_t)(lane / (HV / 4)) * (uint32_t)rv + (uint32_t)c4) * 4u;
                    f32x4 a4, b4;
    #pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        a4[z] = r4[z] * to_f32(p1w[x].v[z]);
                        b4[z] = r4[z] * to_f32(p1v[x].v[z]);
                    }
                    *reinterpret_cast<f32x4*>(at_byte(dv + ro, lo)) = a4;
                    *reinterpret_cast<f32x4*>(at_byte(dw + ro, lo)) = b4;
                }
                if constexpr (G::HL) {
                    put_hl(G::DO, C * LDB, LDB, r, c4, o4);
                    put_hl(G::DR, C * LDB, LDB, r, c4, r4);
                    put_hl(G::UU, C * LDB, LDB, r, c4, u4);
                } else {
                    *reinterpret_cast<f32x4*>(sDO + r * LDV + c4) = o4;
                    *reinterpret_cast<f32x4*>(sDR + r * LDV + c4) = r4;
                    *reinterpret_cast<f32x4*>(sU + r * LDV + c4) = u4;
                }
            }
        };
        const int t0 = n * C;
        const float* Sg = state_of(s_ckpt, n);
        const float* dSg = state_of(ds_ckpt, n);

        // ---- phase 2: X1 = dO S^T, X2 = dR S^T, X3 = U dS'^T over two halves of the value axis;
        // each half of S and dS' goes through registers, loaded one step ahead ----
        f32x4 X1[TPW], X2[TPW], X3[TPW];
    #pragma unroll
        for (int j = 0; j < TPW; ++j) X1[j] = X2[j] = X3[j] = zero4();
    #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            lds_barrier();
            if (hh == 0) {  // every thread is past the previous chunk's reads of these
                if (tid < DK) sXR[tid] = 0.f;
                if (tid == 0) *sFLG = 0;
                p1_use(t0, 0);  // region 1: the previous chunk's q, k, b are read
                p1_load(lane, n, 1);
            }
    #pragma unroll
            for (int i = 0; i < NSH; ++i) {
                const int e = tid + i * NT, r = e / (HV / 4), c4 = (e % (HV / 4)) * 4;
                if constexpr (G::HL) put_hl(G::SH, DK * LDS2, LDS2, r, c4, sv[i]);
                else *reinterpret_cast<f32x4*>(sSH + r * LDH + c4) = sv[i];
            }
            lds_barrier();
            {
                f32x4 acc[2 * TPW];
    #pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    acc[j] = X1[j];
                    acc[TPW + j] = X2[j];
                }
                if constexpr (G::HL)
                    mm_hl<2 * TPW, HV>(acc,
                        [&](int t, int m, int kk, int pl) {
                            return pl_of(t < TPW ? G::DO : G::DR, C * LDB, pl) +
                                   ((it0 + ITS * (t % TPW)) * 16 + m) * LDB + hh * HV + kk;
                        },
                        [&](int, int kk, int nn, int pl) { return pl_of(G::SH, DK * LDS2, pl) + (ct * 16 + nn) * LDS2 + kk; },
                        l16, g4);
                else
                    mm_n<2 * TPW, HV>(acc,
                        [&](int t, int m, int kk) {
                            const float* X = t < TPW ? sDO : sDR;
                            return X[((it0 + ITS * (t % TPW)) * 16 + m) * LDV + hh * HV + kk];
                        },
                        [&](int, int kk, int nn) { return sSH[(ct * 16 + nn) * LDH + kk]; }, l16, g4);
    #pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    X1[j] = acc[j];
                    X2[j] = acc[TPW + j];
                }
            }
            lds_barrier();
    #pragma unroll
            for (int i = 0; i < NSH; ++i) {
                const int e = tid + i * NT, r = e / (HV / 4), c4 = (e % (HV / 4)) * 4;
                const f32x4 d4 = dsv[i], s4 = sv[i];
                if constexpr (G::HL) put_hl(G::SH, DK * LDS2, LDS2, r, c4, d4);
                else *reinterpret_cast<f32x4*>(sSH + r * LDH + c4) = d4;
                const float p = d4[0] * s4[0] + d4[1] * s4[1] + d4[2] * s4[2] + d4[3] * s4[3];
                xd[i] = hh == 0 ? p : xd[i] + p;
            }
            if (hh == 0) {
                load_half(lane, sv, Sg, 1);
                load_half(lane, dsv, dSg, 1);
            }
            lds_barrier();
            if constexpr (G::HL)
                mm_hl<TPW, HV>(X3,
                    [&](int t, int m, int kk, int pl) {
                        return pl_of(G::UU, C * LDB, pl) + ((it0 + ITS * t) * 16 + m) * LDB + hh * HV + kk;
                    },
                    [&](int, int kk, int nn, int pl) { return pl_of(G::SH, DK * LDS2, pl) + (ct * 16 + nn) * LDS2 + kk; },
                    l16, g4);
            else
                mm_n<TPW, HV>(X3, [&](int t, int m, int kk) { return sU[((it0 + ITS * t) * 16 + m) * LDV + hh * HV + kk]; },
                              [&](int, int kk, int nn) { return sSH[(ct * 16 + nn) * LDH + kk]; }, l16, g4);
            if (hh == 0) p1_use(t0, 1);  // the second value half of dO, dR, U (columns no product reads yet)
        }
        // the row sums: the HV / 4 threads of a row are consecutive lanes
    #pragma unroll
        for (int i = 0; i < NSH; ++i) {
    #pragma unroll
            for (int o = 1; o < HV / 4; o <<= 1) xd[i] += __shfl_xor(xd[i], o);
            const int e = tid + i * NT;
            if (e % (HV / 4) == 0) sXD[e / (HV / 4)] = xd[i];
        }
    #pragma unroll
        for (int j = 0; j < TPW; ++j) X2[j] = -X2[j];  // -dR S^T
        lds_barrier();

        // the key-side inputs of the element phase, in flight during phase 3
        const int ec = tid % DK, etb = wave * 64 / DK;  // a wave's threads share a token block
        KeyIn<In, L> in;
        load_key<In, L>(in, q, k, bgate, log_alpha, base_k, ec, rk, t0 + wave * 64 / DK * L, T);

        // ---- phase 3: dA = -dR U^T (j < i), dP = dO U^T (j <= i) ----
        if constexpr (G::HL) {
            // the 20 lower 16 x 16 blocks (I >= J), u < 10 of dA and u >= 10 of dP, block u mod 10
            // in the order (0,0) (1,0) (1,1) (2,0) ...; wave w takes u = w, w + 8, w + 16.  Each
            // value is split once and written twice: into its own triangle of one packed matrix
            // and transposed into the other's
            auto blk = [](int u, int& I, int& J) {
                const int x = u % 10;
                I = x < 1 ? 0 : (x < 3 ? 1 : (x < 6 ? 2 : 3));
                J = x - I * (I + 1) / 2;
            };
            f32x4 acc[3];
    #pragma unroll
            for (int t = 0; t < 3; ++t) acc[t] = zero4();
            mm_hl<3, DV>(acc,
                [&](int t, int m, int kk, int pl) {
                    const int u = min(wave + 8 * t, 19);
                    int I, J;
                    blk(u, I, J);
                    return pl_of(u >= 10 ? G::DO : G::DR, C * LDB, pl) + (I * 16 + m) * LDB + kk;
                },
                [&](int t, int kk, int nn, int pl) {
                    const int u = min(wave + 8 * t, 19);
                    int I, J;
                    blk(u, I, J);
                    return pl_of(G::UU, C * LDB, pl) + (J * 16 + nn) * LDB + kk;
                }, l16, g4);
            bf16* m1h = reinterpret_cast<bf16*>(smem + G::M1H);
            bf16* m2h = reinterpret_cast<bf16*>(smem + G::M2H);
            constexpr int PL = G::PM / 2;  // elements from a hi plane to its lo plane
    #pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int u = wave + 8 * t;
                if (u >= 20) continue;
                int I, J;
                blk(u, I, J);
                const bool isP = u >= 10;
                const int jj = J * 16 + l16, i0 = I * 16 + 4 * g4;
                f32x4 x = isP ? acc[t] : -acc[t];
                bf16x4 h, l;
                split_hl(x, h, l);
                bf16* own = isP ? m1h : m2h;  // dP into M1 (j <= i), dA into M2 (j < i)
                bf16* oth = isP ? m2h : m1h;  // transposed: dP^T into M2, dA^T into M1
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (isP ? jj <= i0 + r : jj < i0 + r) {
                        own[(i0 + r) * G::LDM + jj] = h[r];
                        own[(i0 + r) * G::LDM + jj + PL] = l[r];
                    }
                }
                if (I > J) {  // the transposed block lies wholly in the other triangle
                    *reinterpret_cast<bf16x4*>(oth + jj * G::LDM + i0) = h;
                    *reinterpret_cast<bf16x4*>(oth + jj * G::LDM + i0 + PL) = l;
                } else {
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (isP ? jj <= i0 + r : jj < i0 + r) {
                            oth[jj * G::LDM + i0 + r] = h[r];
                            oth[jj * G::LDM + i0 + r + PL] = l[r];
                        }
                    }
                }
            }
        } else {
            // wave w: block pairs p = w and w + 8, (I, J) = (p / 4, p % 4), both dA and dP; zero
            // above the diagonal
            f32x4 acc[4];
    #pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = zero4();
            mm_n<4, DV>(acc,
                [&](int t, int m, int kk) {
                    const int p = wave + 8 * (t >> 1);
                    return (t & 1 ? sDO : sDR)[((p >> 2) * 16 + m) * LDV + kk];
                },
                [&](int t, int kk, int nn) {
                    const int p = wave + 8 * (t >> 1);
                    return sU[((p & 3) * 16 + nn) * LDV + kk];
                }, l16, g4);
    #pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int p = wave + 8 * (t >> 1), I = p >> 2, J = p & 3, mat = t & 1;
                float* dst = mat ? sDP : sDA;
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = I * 16 + g4 * 4 + r, jj = J * 16 + l16;
                    const bool keep = mat ? (jj <= i) : (jj < i);
                    dst[i * LDC + jj] = keep ? (mat ? acc[t][r] : -acc[t][r]) : 0.f;
                }
            }
        }
        lds_barrier();  // region 1 (dO, dR, U) is free from here on

        // element phase: G (chunk-local cumulative log alpha) and the raw q, k, b of the chunk
        {
            float x[L];
            float run = 0.f;
    #pragma unroll
            for (int m = 0; m < L; ++m) {
                run += FULL || t0 + etb * L + m < T ? in.g[m] : 0.f;
                x[m] = run;
            }
            sTOT[etb * DK + ec] = run;
            lds_barrier();
            float tot = 0.f, after = 0.f, oh = 0.f, ol = 0.f;
    #pragma unroll
            for (int j = 0; j < TB; ++j) {
                const float vj = sTOT[j * DK + ec];
                tot += vj;
                if (j < etb) {
                    float sv, ev;
                    two_sum(oh, vj, sv, ev);
                    oh = sv;
                    ol += ev;
                }
                if (j > etb) after += vj;
            }
            sOFH[etb * DK + ec] = oh;
            sOFL[etb * DK + ec] = ol;
            sAFT[etb * DK + ec] = after;
            if (etb == 0) {
                sGC[ec] = exp_any(tot);
                if (!(tot >= kMildLog)) *sFLG = 1;
            }
    #pragma unroll
            for (int m = 0; m < L; ++m) {
                const int i = etb * L + m, t = t0 + i;
                In qv = from_f32<In>(0.f), kv = qv, bv = qv;
                if (FULL || t < T) {
                    qv = in.q[m];
                    kv = in.k[m];
                    bv = in.b[m];
                }
                sG[i * LDF + ec] = x[m];  // block-local
                sQ[i * LDT + ec] = qv;
                sK[i * LDT + ec] = kv;
                sB[i * LDT + ec] = bv;
            }
        }
        lds_barrier();
        const bool mild = *sFLG == 0;

        // the G_C term of U dS'^T: sum_i k_ic e^{G_C - G_ic} X3_ic
        {
            float part = 0.f;
    #pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int it = it0 + ITS * j;
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = it * 16 + g4 * 4 + r;
                    part += to_f32(sK[i * LDT + c]) * exp_any(Gsuf(i, c)) * X3[j][r];
                }
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            if (g4 == 0) atomicAdd(sXR + c, part);
        }

        // ---- phase 4: the masked decay products; afterwards X1 = dq, X2 = d(kh), X3 = dk through
        // the decays (without b.d(kh)) ----
        if (mild) {
            const float gc = sGC[c];
    #pragma unroll
            for (int j = 0; j < TPW; ++j) X3[j] *= gc;
            if constexpr (G::HL) {
                // bf16 hi/lo products over blocks of 32 contraction tokens: lane group g4 takes
                // the tokens 32 b + 8 g4 + e (e = 0..7), its factors for those eight at once and
                // the dP, dA rows of X1, X2 as two 16-byte reads; a block on the zero side of
                // the diagonal for a row tile is skipped
    #pragma unroll
                for (int b32 = 0; b32 < C / 32; ++b32) {
                    float ki[8], kg[8], qg[8];
    #pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int r = b32 * 32 + 8 * g4 + e;
                        const float Gr = Gof(r, c);
                        const float kr = to_f32(sK[r * LDT + c]);
                        const float ep = exp_any(Gr), en = exp_any(-Gr);
                        ki[e] = kr * en;                                // k / Gamma
                        kg[e] = to_f32(sB[r * LDT + c]) * kr * ep;      // kh.Gamma
                        qg[e] = to_f32(sQ[r * LDT + c]) * ep;           // q.Gamma
                    }
                    bf16x8 kih, kil, kgh, kgl, qgh, qgl;
                    split_hl8(ki, kih, kil);
                    split_hl8(kg, kgh, kgl);
                    split_hl8(qg, qgh, qgl);
    #pragma unroll
                    for (int j = 0; j < TPW; ++j) {
                        const int it = it0 + ITS * j;
                        // row i of M1 and M2 over this lane's eight tokens: below the diagonal M1 is
                        // dP and M2 dA (X1, X2), above it M1 is dA^T and M2 dP^T (X3)
                        const int row = (it * 16 + l16) * G::LDM + b32 * 32 + 8 * g4;
                        const bf16* pm = reinterpret_cast<const bf16*>(smem + G::M1H) + row;
                        const bf16x8 m1h = *reinterpret_cast<const bf16x8*>(pm);
                        const bf16x8 m1l = *reinterpret_cast<const bf16x8*>(pm + G::PM / 2);
                        const bf16x8 m2h = *reinterpret_cast<const bf16x8*>(pm + G::PM);
                        const bf16x8 m2l = *reinterpret_cast<const bf16x8*>(pm + 3 * G::PM / 2);
                        if (2 * b32 == (it & ~1)) {
                            // the block on the diagonal: tokens r <= i (e <= n) to X1, r < i to X2
                            const int n = it * 16 + l16 - b32 * 32 - 8 * g4;
                            bf16x8 p1h, p1l, a1h, a1l, a2h, a2l, p2h, p2l;
                            take_first(m1h, n + 1, p1h, a1h);
                            take_first(m1l, n + 1, p1l, a1l);
                            take_first(m2h, n, a2h, p2h);
                            take_first(m2l, n, a2l, p2l);
                            X1[j] = mf32(X1[j], p1h, kih);
                            X2[j] = mf32(X2[j], a2h, kih);
                            X1[j] = mf32(X1[j], p1h, kil);
                            X2[j] = mf32(X2[j], a2h, kil);
                            X1[j] = mf32(X1[j], p1l, kih);
                            X2[j] = mf32(X2[j], a2l, kih);
                            X3[j] = mf32(X3[j], a1h, kgh);
                            X3[j] = mf32(X3[j], a1h, kgl);
                            X3[j] = mf32(X3[j], a1l, kgh);
                            X3[j] = mf32(X3[j], p2h, qgh);
                            X3[j] = mf32(X3[j], p2h, qgl);
                            X3[j] = mf32(X3[j], p2l, qgh);
                        } else if (2 * b32 < it) {  // wholly below: X1, X2
                            X1[j] = mf32(X1[j], m1h, kih);
                            X2[j] = mf32(X2[j], m2h, kih);
                            X1[j] = mf32(X1[j], m1h, kil);
                            X2[j] = mf32(X2[j], m2h, kil);
                            X1[j] = mf32(X1[j], m1l, kih);
                            X2[j] = mf32(X2[j], m2l, kih);
                        } else {  // wholly above: X3
                            X3[j] = mf32(X3[j], m1h, kgh);
                            X3[j] = mf32(X3[j], m1h, kgl);
                            X3[j] = mf32(X3[j], m1l, kgh);
                            X3[j] = mf32(X3[j], m2h, qgh);
                            X3[j] = mf32(X3[j], m2h, qgl);
                            X3[j] = mf32(X3[j], m2l, qgh);
                        }
                    }
                }
            } else {
                // blocks of 16 contraction tokens; lane group g4 takes the tokens 16 b + 4 g4 + s of
                // block b at the four MFMA steps s (its factors for four tokens at once, and the dP, dA
                // rows of X1, X2 as 16-byte reads)
        #pragma unroll
                for (int b16 = 0; b16 < C / 16; ++b16) {
                    float ki[4], kg[4], qg[4];
        #pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int r = b16 * 16 + 4 * g4 + s;
                        const float Gr = Gof(r, c);
                        const float kr = to_f32(sK[r * LDT + c]);
                        const float ep = exp_any(Gr), en = exp_any(-Gr);
                        ki[s] = kr * en;                                // k / Gamma
                        kg[s] = to_f32(sB[r * LDT + c]) * kr * ep;      // kh.Gamma
                        qg[s] = to_f32(sQ[r * LDT + c]) * ep;           // q.Gamma
                    }
        #pragma unroll
                    for (int j = 0; j < TPW; ++j) {
                        const int it = it0 + ITS * j;
                        if (b16 <= it) {  // X1, X2: tokens up to i (dP, dA are zero above the diagonal)
                            const f32x4 p4 = *reinterpret_cast<const f32x4*>(sDP + (it * 16 + l16) * LDC + b16 * 16 + 4 * g4);
                            const f32x4 a4 = *reinterpret_cast<const f32x4*>(sDA + (it * 16 + l16) * LDC + b16 * 16 + 4 * g4);
        #pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                X1[j] = mfma4(X1[j], p4[s], ki[s]);
                                X2[j] = mfma4(X2[j], a4[s], ki[s]);
                            }
                        }
                        if (b16 >= it) {  // X3: tokens from i on
        #pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const int r = b16 * 16 + 4 * g4 + s;
                                X3[j] = mfma4(X3[j], sDA[r * LDC + it * 16 + l16], kg[s]);
                                X3[j] = mfma4(X3[j], sDP[r * LDC + it * 16 + l16], qg[s]);
                            }
                        }
                    }
                }
            }
    #pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int it = it0 + ITS * j;
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float Gi = Gof(it * 16 + g4 * 4 + r, c);
                    const float ep = exp_any(Gi);
                    X1[j][r] *= ep;
                    X2[j][r] *= ep;
                    X3[j][r] *= exp_any(-Gi);
                }
            }
        } else {
    #pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int it = it0 + ITS * j;
                for (int r = 0; r < 4; ++r) {
                    const int i = it * 16 + g4 * 4 + r;
                    float sq = 0.f, sh = 0.f, sk = 0.f;
                    // dP[i][jj], dA[i][jj] (jj <= i) and dA[ii][i], dP[ii][i] (ii >= i)
                    auto dp_row = [&](int jj) {
                        if constexpr (G::HL) return pk(G::M1H, i, jj);
                        else return sDP[i * LDC + jj];
                    };
                    auto da_row = [&](int jj) {
                        if constexpr (G::HL) return jj < i ? pk(G::M2H, i, jj) : 0.f;
                        else return sDA[i * LDC + jj];
                    };
                    auto da_col = [&](int ii) {
                        if constexpr (G::HL) return ii > i ? pk(G::M1H, i, ii) : 0.f;
                        else return sDA[ii * LDC + i];
                    };
                    auto dp_col = [&](int ii) {
                        if constexpr (G::HL) return pk(G::M2H, i, ii);
                        else return sDP[ii * LDC + i];
                    };
                    for (int jj = 0; jj <= i; ++jj) {
                        const float f = exp_any(Gdiff(i, jj, c)) * to_f32(sK[jj * LDT + c]);
                        sq += dp_row(jj) * f;
                        sh += da_row(jj) * f;
                    }
                    for (int ii = i; ii < C; ++ii) {
                        const float f = exp_any(Gdiff(ii, i, c));
                        const float kh = to_f32(sB[ii * LDT + c]) * to_f32(sK[ii * LDT + c]);
                        sk += (da_col(ii) * kh + dp_col(ii) * to_f32(sQ[ii * LDT + c])) * f;
                    }
                    const float ep = exp_any(Gof(i, c));
                    X1[j][r] = ep * X1[j][r] + sq;
                    X2[j][r] = ep * X2[j][r] + sh;
                    X3[j][r] = exp_any(Gsuf(i, c)) * X3[j][r] + sk;
                }
            }
        }
        lds_barrier();  // dA, dP are consumed: region 2 takes dG
        {  // the next chunk's first loads (the last chunk reloads its own: no branch, see the serial
           // kernels), into registers free since phase 2
            const int nn = min(n + 1, n1 - 1);
            p1_load(lane, nn, 0);
            load_half(lane, sv, state_of(s_ckpt, nn), 0);
            load_half(lane, dsv, state_of(ds_ckpt, nn), 0);
        }

        // ---- phase 5: dq, dk, db; the per-token decay gradient dG ----
        // stores at a wave-uniform row base plus a 32-bit lane offset (row 4 g4 + r of the tile)
        const uint32_t lo5 = ((uint32_t)(4 * g4) * (uint32_t)rk + (uint32_t)c) * 4u;
        float dgv[TPW][4];
    #pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int it = it0 + ITS * j;
    #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = it * 16 + g4 * 4 + r, t = t0 + i;
                const float qv = to_f32(sQ[i * LDT + c]), kv = to_f32(sK[i * LDT + c]), bv = to_f32(sB[i * LDT + c]);
                const float dqv = X1[j][r], dkh = X2[j][r];
                const float dkv = X3[j][r] + bv * dkh;
                dgv[j][r] = qv * dqv + 2.f * bv * kv * dkh - kv * dkv;
                if constexpr (KT != 8) sDG[i * LDF + c] = dgv[j][r];
                if (FULL || t < T) {
                    const int64_t ro = base_k + (int64_t)(t0 + it * 16 + r) * rk;
                    *at_byte(dq + ro, lo5) = dqv;
                    *at_byte(dk + ro, lo5) = dkv;
                    *at_byte(db + ro, lo5) = kv * dkh;
                }
            }
        }
        // reverse cumulative sum over the chunk, plus the G_C terms
        if constexpr (KT == 8) {
            // a wave holds all 64 tokens of its 16 channels (row tiles j, lane group g4 has tokens
            // 16 j + 4 g4 + r): the sum runs in registers, over the lane's four tokens of a tile and
            // across the four lane groups of the channel (lanes 16 apart)
            float after = sXR[c] + sGC[c] * sXD[c];  // complete since the barrier after phase 4
    #pragma unroll
            for (int j = TPW - 1; j >= 0; --j) {
                const float sj = (dgv[j][0] + dgv[j][1]) + (dgv[j][2] + dgv[j][3]);
                const float s1 = __shfl_xor(sj, 16), s2 = __shfl_xor(sj, 32), s3 = __shfl_xor(sj, 48);
                // the lane groups after g4: for g4 = 0 all three, 1: g4 ^ 2 and g4 ^ 3, 2: g4 ^ 1
                const float later = g4 == 0 ? (s1 + s2) + s3 : (g4 == 1 ? s2 + s3 : (g4 == 2 ? s1 : 0.f));
                float run = after + later;
    #pragma unroll
                for (int r = 3; r >= 0; --r) {
                    run += dgv[j][r];
                    if (FULL || t0 + j * 16 + 4 * g4 + r < T)
                        *at_byte(dg + base_k + (int64_t)(t0 + j * 16 + r) * rk, lo5) = run;
                }
                after += (sj + s1) + (s2 + s3);
            }
        } else {
            lds_barrier();
            float run = 0.f;
    #pragma unroll
            for (int m = L - 1; m >= 0; --m) run += sDG[(etb * L + m) * LDF + ec];
            sTOT[etb * DK + ec] = run;
            lds_barrier();
            float after = sXR[ec] + sGC[ec] * sXD[ec];
    #pragma unroll
            for (int j = 0; j < TB; ++j)
                if (j > etb) after += sTOT[j * DK + ec];
            run = after;
    #pragma unroll
            for (int m = L - 1; m >= 0; --m) {
                const int i = etb * L + m, t = t0 + i;
                run += sDG[i * LDF + ec];
                if (FULL || t < T) *at_byte(dg + base_k + (int64_t)t * rk, (uint32_t)ec * 4u) = run;
            }
        }
    };
    const int nfull = min(n1, T / C);  // chunks n0 .. nfull - 1 are full
    for (int n = n0; n < nfull; ++n) chunk(n, std::true_type{});
    if (nfull < n1) chunk(n1 - 1, std::false_type{});  // the sequence's last, partial chunk
}


template <typename In, int D>
hipError_t launch_grad(const BwdArgs& a) {
    // runs of consecutive chunks, about one workgroup per compute unit
    const int64_t bh = a.B * a.H, nch = (a.T + C - 1) / C;
    const int64_t cus = a.cus > 0 ? a.cus : 1;
    const int64_t nper = (bh * nch + cus - 1) / cus;
    const int64_t ngrp = (nch + nper - 1) / nper;
    hipLaunchKernelGGL((bwd_chunk_kernel<In, D, D>), dim3((unsigned)(bh * ngrp)), dim3(NT), 0,
                       (hipStream_t)a.stream, (const In*)a.q, (const In*)a.k, (const In*)a.v, a.log_alpha,
                       (const In*)a.b, (const In*)a.w, a.d_o, a.s_ckpt, a.ds_ckpt, a.u, a.dr, a.g_q, a.g_k,
                       a.g_v, a.g_log_alpha, a.g_b, a.g_w, (int)a.T, (int)a.H, (int)nper);
    return hipGetLastError();
}

template <typename In, int D>
hipError_t launch_bwd_typed(const BwdArgs& a) {
    const int64_t bh = a.B * a.H, nch = (a.T + C - 1) / C;
    // kernel 0: runs of consecutive chunks, about one workgroup per compute unit
    const int64_t cus = a.cus > 0 ? a.cus : 1;
    const int64_t nper = (bh * nch + cus - 1) / cus;
    const int64_t ngrp = (nch + nper - 1) / nper;
    hipLaunchKernelGGL((bwd_local_kernel<In, D, D>), dim3((unsigned)(bh * ngrp)), dim3(NT), 0, (hipStream_t)a.stream,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, a.log_alpha, (const In*)a.b, (const In*)a.w,
                       a.loc, (int)a.T, (int)a.H, (int)nper);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // bf16 inputs: the serial passes' products on bf16 hi/lo operands; fp32 inputs: fp32
    constexpr bool HL = sizeof(In) == 2;
    const unsigned nser = (unsigned)(bh * SerCfg<D, D>::NSL);
    hipLaunchKernelGGL((bwd_fwd_kernel<D, D, HL>), dim3(nser), dim3(NT), 0, (hipStream_t)a.stream, a.loc,
                       a.initial_state, a.s_ckpt, a.u, (int)a.T, (int)a.H, (int)bh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_state_kernel<D, D, HL>), dim3(nser), dim3(NT), 0, (hipStream_t)a.stream, a.loc, a.d_o,
                       a.d_final_state, a.ds_ckpt, a.dr, a.g_s0, (int)a.T, (int)a.H, (int)bh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_grad<In, D>(a);
}

}  // namespace bw

hipError_t launch_chunk_bwd(const BwdArgs& a) {
    if (a.dk != a.dv) return hipErrorInvalidValue;
    if (a.dtype_bf16) {
        if (a.dk == 128) return bw::launch_bwd_typed<bf16, 128>(a);
        if (a.dk == 64) return bw::launch_bwd_typed<bf16, 64>(a);
    } else if (a.dk == 64) {
        return bw::launch_bwd_typed<float, 64>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn2
