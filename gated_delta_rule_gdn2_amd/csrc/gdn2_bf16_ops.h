// gdn2_bf16_ops.h -- device pieces shared by the bf16 chunk kernels (gfx950): hi / lo bf16
// splits, LDS stores and barriers, the unit-lower-triangular inverse by doubling, and the
// decay-pivoted A and P of a strong-decay chunk.  Included by the fused forward and by the
// split forward's chunk-local kernel; they differ in LDS layout (the template parameter G)
// and in where P goes (a store functor).
#pragma once

#include "gdn2_device.h"

namespace gdn2 {
namespace cb {

constexpr int C = 64;

__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
    hi = (bf16)x;
    lo = (bf16)(x - (float)hi);
}

template <int N>
__device__ __forceinline__ void store_bf16(bf16* p, const float (&x)[N]) {
    typedef bf16 V __attribute__((ext_vector_type(N)));
    V y;
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = (bf16)x[i];
    *reinterpret_cast<V*>(__builtin_assume_aligned(p, 2 * N < 16 ? 2 * N : 16)) = y;
}

template <int N>
__device__ __forceinline__ void store_bf16_split(bf16* hi, bf16* lo, const float (&x)[N]) {
    typedef bf16 V __attribute__((ext_vector_type(N)));
    V h, l;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        bf16 a, b;
        split_bf16(x[i], a, b);
        h[i] = a;
        l[i] = b;
    }
    *reinterpret_cast<V*>(__builtin_assume_aligned(hi, 2 * N < 16 ? 2 * N : 16)) = h;
    *reinterpret_cast<V*>(__builtin_assume_aligned(lo, 2 * N < 16 ? 2 * N : 16)) = l;
}

__device__ __forceinline__ void acc_to_array(const f32x4& a, float (&x)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = a[r];
}

// hi / lo K = 16 operands of an accumulator
struct Split16 { Frag16<bf16> hi, lo; };
__device__ __forceinline__ Split16 split16(const f32x4& a) {
    Split16 s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16 h, l;
        split_bf16(a[e], h, l);
        s.hi.v[e] = h;
        s.lo.v[e] = l;
    }
    return s;
}

// hi / lo K = 32 operands of an accumulator pair (permuted slot map)
struct Split32 { Frag<bf16> hi, lo; };
__device__ __forceinline__ Split32 split32(const f32x4& a, const f32x4& b) {
    Split32 s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16 h, l;
        split_bf16(a[e], h, l);
        s.hi.v[e] = h;
        s.lo.v[e] = l;
        split_bf16(b[e], h, l);
        s.hi.v[e + 4] = h;
        s.lo.v[e + 4] = l;
    }
    return s;
}

// Column position inside a transposed [channel][token] bf16 tile: 16-byte units (8 tokens) are
// XOR-swizzled by (row / 16) % 8 so that the element phase's stores to rows 8 apart hit distinct
// banks; 16 consecutive rows share one swizzle value.
__device__ __forceinline__ int swz(int row, int col) {
    return (((col >> 3) ^ ((row >> 4) & 7)) << 3) | (col & 7);
}

// N elements at a byte offset from a base (the base is uniform across the workgroup and
// lives in scalar registers; the offset is a 32-bit per-lane value)
template <typename T, int N>
__device__ __forceinline__ Vec<T, N> gload(const void* base, uint32_t byte_off) {
    return load_vec<T, N>(reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off));
}

// N elements of T (bf16 or float) as loaded: raw 32-bit words, each element widened to fp32 where
// it is used.  Inputs loaded for the next chunk are carried across the chunk loop in this form: a
// bf16 vector carried element by element is unpacked, one register per element, at the bottom of
// the loop, which makes every wave wait there for all of its loads and stores.
template <typename T, int N>
struct Raw {
    static_assert((N * sizeof(T)) % 4 == 0, "whole 32-bit words");
    static constexpr int W = N * (int)sizeof(T) / 4;
    uint32_t u[W];
    __device__ __forceinline__ float f(int i) const {
        if constexpr (sizeof(T) == 4) {
            return __uint_as_float(u[i]);
        } else {
            // bf16 -> fp32: the 16 bits become the high half of the fp32 pattern
            return __uint_as_float((i & 1) ? (u[i >> 1] & 0xffff0000u) : (u[i >> 1] << 16));
        }
    }
};

template <typename T, int N>
__device__ __forceinline__ Raw<T, N> gload_raw(const void* base, uint32_t byte_off) {
    constexpr int W = Raw<T, N>::W;
    const char* p = reinterpret_cast<const char*>(base) + byte_off;
    Raw<T, N> r;
    if constexpr (W == 1) {
        r.u[0] = *reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
    } else {
        typedef uint32_t V __attribute__((ext_vector_type(W)));
        const V x = *reinterpret_cast<const V*>(__builtin_assume_aligned(p, W * 4));
#pragma unroll
        for (int i = 0; i < W; ++i) r.u[i] = x[i];
    }
    return r;
}

// A buffer resource over `bytes` bytes from `base`: loads past the end read zeros and stores
// past the end are dropped
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// N elements of T at a byte offset into a buffer resource (zeros past its end)
template <typename T, int N>
__device__ __forceinline__ Raw<T, N> bload_raw(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    constexpr int W = Raw<T, N>::W;
    Raw<T, N> x;
    if constexpr (W == 1) {
        x.u[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0);
    } else if constexpr (W == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0);
        x.u[0] = v[0];
        x.u[1] = v[1];
    } else {
        static_assert(W == 4, "1, 2 or 4 words");
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) x.u[i] = v[i];
    }
    return x;
}

// Workgroup barrier for data exchanged through LDS only: waits for this wave's LDS accesses,
// not for its global loads, so the next chunk's loads stay in flight across it (a full
// __syncthreads() would drain them).  Waves never exchange data through global memory.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// keep the instructions before and after apart (all fragment loads are issued before the
// MFMAs that consume them, so their latencies overlap)
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// A lane-dependent LDS byte offset that the compiler may not hoist out of the chunk loop: every
// phase derives its addresses from one such base plus constant offsets (which fold into the
// instructions' offset field), instead of keeping one register per address live across the loop.
__device__ __forceinline__ int opq(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// acc + X Y for 16 x 16 matrices, with both factors as hi + lo bf16 pairs (three bf16 MFMAs;
// the lo * lo term, below 2^-16 of the product, is dropped).  xt: X^T in accumulator layout
// (lane (m, g) holds X[m][4g + r]); y: Y in accumulator layout (lane (n, g) holds Y[4g + r][n]).
__device__ __forceinline__ f32x4 mm16s(f32x4 acc, const Split16& xt, const Split16& y) {
    mma16(acc, xt.hi, y.hi);
    mma16(acc, xt.hi, y.lo);
    mma16(acc, xt.lo, y.hi);
    return acc;
}

// (I + N)^{-1} for a strictly lower triangular 16 x 16 N.  N is nilpotent (N^16 = 0), so
// the inverse is the finite sum of (-N)^n, n < 16, which factors as
// (I - N)(I + N^2)(I + N^4)(I + N^8).  nt: lane (i, g) holds N[i][4g + r]; n: lane (j, g)
// holds N[4g + r][j].  Returns T = (I + N)^{-1} as lane (i, g) holding T[i][4g + r]; the
// products carry about 16 significant bits, more than the bf16 T they feed.
__device__ __forceinline__ f32x4 unit_lower_inverse(const f32x4& nt, const f32x4& n, int l16, int g4) {
    const Split16 s1t = split16(nt), s1 = split16(n);
    const f32x4 n2 = mm16s(zero4(), s1t, s1);   // N^2
    const f32x4 n2t = mm16s(zero4(), s1, s1t);  // (N^2)^T
    const Split16 s2 = split16(n2), s2t = split16(n2t);
    const f32x4 n4 = mm16s(zero4(), s2t, s2);   // N^4
    const f32x4 n4t = mm16s(zero4(), s2, s2t);  // (N^4)^T
    const Split16 s4 = split16(n4), s4t = split16(n4t);
    const Split16 s8 = split16(mm16s(zero4(), s4t, s4));  // N^8
    // t holds T_m^T in accumulator layout; T_2m^T = T_m^T + (N^2m)^T T_m^T
    f32x4 t;
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = (4 * g4 + r == l16 ? 1.f : 0.f) - nt[r];
    t = mm16s(t, s2, split16(t));
    t = mm16s(t, s4, split16(t));
    t = mm16s(t, s8, split16(t));
    return t;
}

// A and P of a strong-decay chunk (some channel's whole-chunk decay is below 2^-64): the
// chunk is split recursively at midpoints, and every pair (i, j) is formed at the level
// whose split point p it straddles, as Gamma_{i<-p} Gamma_{p<-j} with both factors <= 1.
// Levels 64 and 32 span blocks and read the group tiles the element phase wrote to the
// work area; levels 16 to 2 and P's diagonal lie inside one 16-token block and are formed
// here from the inputs (reloaded, they are in L2).  Ends by inverting I + A_II by
// doubling, like the mild path.
// Diagonal block I of T = (I + A)^{-1} from its transposed accumulator t (lane (i, g) holds
// T_II[i][4 g + r]): rows into T, columns into T^T, and zeros into the block right of it for
// I = 0, 2 (the K = 32 products over T read blocks (0,1) and (2,3)).
template <typename G>
__device__ __forceinline__ void store_tdiag(char* smem, int I, int l16, int g4, const f32x4& t) {
    constexpr int LC = G::LC;
    float x[4];
    acc_to_array(t, x);
    bf16* row = reinterpret_cast<bf16*>(smem + G::TR + ((I * 16 + l16) * LC + I * 16 + g4 * 4) * 2);
    store_bf16<4>(row, x);
    if ((I & 1) == 0) {
        // zeros made here: a zero pair kept in registers from the top of the kernel is what the
        // register allocator spills first, and its reload would wait for every load in flight
        uint32_t z0, z1;
        asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0" : "=v"(z0), "=v"(z1));
        *reinterpret_cast<uint2*>(row + 16) = make_uint2(z0, z1);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<bf16*>(smem + G::TTR + ((I * 16 + g4 * 4 + r) * LC + I * 16 + l16) * 2) = (bf16)x[r];
}

// G: the LDS layout (RX work rows of G::LDK bf16, AM, TR, TTR of G::LC); Src: the inputs of
// this lane's token slot m (token 16 I + 4 ts + m, channels c0 .. c0 + CPL - 1),
// src(m, decay, q, k, b) fills four float[CPL] arrays -- read from global memory, or handed over
// from the registers the element phase loaded them into; PutP: stores a row segment of P, put_p(row, col, p[4]) for
// P[row][col .. col + 3]; PutT: receives each diagonal block of T in fp32 as well, put_t(I, t)
// with lane (i, g) of t holding T_II[i][4 g + r].
template <typename G, int DK, typename Gt, typename Src, typename PutP, typename PutT>
__device__ __forceinline__ void strong_ap_body(char* smem, Src src, int ntok, PutP put_p, PutT put_t) {
    constexpr int CPL = DK / 32, LDK = G::LDK, LC = G::LC;
    bf16* sX = reinterpret_cast<bf16*>(smem + G::RX);
    bf16* sA = reinterpret_cast<bf16*>(smem + G::AM);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int I = wave & 3, hf = wave >> 2, ts = lane >> 4;
    const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
    // ---- level 64 (pairs (2,0) (2,1) (3,0) (3,1)) and level 32 ((1,0) (3,2)): one pair per wave ----
    if (wave < 6) {
        int Ib, Jb, ga, gp, gcol;
        if (wave < 4) {
            Ib = wave < 2 ? 2 : 3;
            Jb = wave & 1;
            ga = Ib - 2; gp = Ib; gcol = 4 + Jb;
        } else {
            Ib = wave == 4 ? 1 : 3;
            Jb = Ib - 1;
            ga = 6 + Ib / 2; gp = 8 + Ib / 2; gcol = 10 + Jb / 2;
        }
        f32x4 accA = zero4(), accP = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const int kc = kk * 32 + g4 * 8;
            const Frag<bf16> fk = load_contig(sX + (gcol * 16 + l16) * LDK + kc);
            const Frag<bf16> fa = load_contig(sX + (ga * 16 + l16) * LDK + kc);
            const Frag<bf16> fq = load_contig(sX + (gp * 16 + l16) * LDK + kc);
            mma(accA, fk, fa);
            mma(accP, fk, fq);
        }
        float a[4], p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) { a[r] = -accA[r]; p[r] = accP[r]; }
        const int idx = (Ib * 16 + l16) * LC + Jb * 16 + g4 * 4;
        store_bf16<4>(sA + idx, a);
        put_p(Ib * 16 + l16, Jb * 16 + g4 * 4, p);
    }
    // ---- levels 16, 8, 4, 2 inside block I, then P's diagonal ----
    // decays of this lane's tokens, and the 4-token product of the token slot ts ^ 1
    // and this lane's q, k and b.k (zero past the end of the sequence), read once for all levels
    float al[CPL][4], x16[CPL];
    float tq[4][CPL], tk[4][CPL], tb[4][CPL];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = I * 16 + ts * 4 + m;
        const bool valid = i < ntok;
        float g[CPL], xq[CPL], xk[CPL], xb[CPL];
        src(m, g, xq, xk, xb);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            al[c][m] = valid ? Gt::alpha(g[c]) : 1.f;
            tq[m][c] = valid ? xq[c] : 0.f;
            tk[m][c] = valid ? xk[c] : 0.f;
            tb[m][c] = valid ? Gt::gate(xb[c]) * xk[c] : 0.f;
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) x16[c] = __shfl_xor(al[c][0] * al[c][1] * al[c][2] * al[c][3], 16);
    lds_barrier();  // the level tiles below reuse the group-tile rows
    // Each wave forms the products of its own channel half (the contraction splits over channels,
    // and every level's masked sum is linear), so a level needs no barrier: the wave writes its
    // half of the block's level tiles and reads back only that half.  Waves I and I + 4 then sum
    // their partial products once.
    bf16* lv = sX + (I * 48) * LDK;  // rows: [0,16) A rows, [16,32) P rows, [32,48) columns
    f32x4 dA = zero4(), dAn = zero4(), dP = zero4();
#pragma unroll
    for (int L = 0; L < 5; ++L) {
        const int size = L < 4 ? (16 >> L) : 1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = ts * 4 + m;  // token within the block
            // split point p of the segment of i (last token of its lower half); a token in the
            // upper half is a row with factor Gamma_{i<-p}, one in the lower half a column with
            // factor Gamma_{p<-i}; both are products of at most one lane's decays and x16
            bool row = false;
            float f[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float lpm = m == 0 ? al[c][0] : m == 1 ? al[c][0] * al[c][1]
                                : m == 2 ? al[c][0] * al[c][1] * al[c][2]
                                         : al[c][0] * al[c][1] * al[c][2] * al[c][3];
                const float lsm = m == 3 ? 1.f : m == 2 ? al[c][3] : m == 1 ? al[c][2] * al[c][3]
                                                                    : al[c][1] * al[c][2] * al[c][3];
                if (L == 0) {         // p = 7
                    row = ts >= 2;
                    f[c] = row ? (ts == 3 ? x16[c] : 1.f) * lpm : lsm * (ts == 0 ? x16[c] : 1.f);
                } else if (L == 1) {  // p = 3, 11
                    row = ts & 1;
                    f[c] = row ? lpm : lsm;
                } else if (L == 2) {  // p = 4 ts + 1
                    row = m >= 2;
                    f[c] = row ? (m == 2 ? al[c][2] : al[c][2] * al[c][3]) : (m == 1 ? 1.f : al[c][1]);
                } else if (L == 3) {  // p = 4 ts + 2 (m / 2)
                    row = m & 1;
                    f[c] = row ? al[c][m] : 1.f;
                } else {
                    f[c] = 1.f;
                }
            }
            float ra[CPL], rp[CPL], cl[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float qv = tq[m][c], kv = tk[m][c], bk = tb[m][c];
                if (L == 4) {
                    ra[c] = 0.f; rp[c] = qv; cl[c] = kv;
                } else {
                    ra[c] = row ? bk * f[c] : 0.f;
                    rp[c] = row ? qv * f[c] : 0.f;
                    cl[c] = row ? 0.f : kv * f[c];
                }
            }
            store_bf16<CPL>(lv + i * LDK + c0, ra);
            store_bf16<CPL>(lv + (16 + i) * LDK + c0, rp);
            store_bf16<CPL>(lv + (32 + i) * LDK + c0, cl);
        }
        // the wave's own writes before its reads (LDS keeps one wave's accesses in order)
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // tA: lane holds A[l16][4 g4 + r] of the block over this channel half; tAn: A[4 g4 + r][l16];
        // tP like tA
        f32x4 tA = zero4(), tAn = zero4(), tP = zero4();
#pragma unroll
        for (int k2 = 0; k2 < DK / 64; ++k2) {
            const int kc = (hf * (DK / 64) + k2) * 32 + g4 * 8;
            const Frag<bf16> fk = load_contig(lv + (32 + l16) * LDK + kc);
            const Frag<bf16> fq = load_contig(lv + (16 + l16) * LDK + kc);
            mma(tP, fk, fq);
            if (L < 4) {
                const Frag<bf16> fa = load_contig(lv + l16 * LDK + kc);
                mma(tA, fk, fa);
                mma(tAn, fa, fk);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = l16, j = g4 * 4 + r;
            const bool keep = L < 4 ? (i / size == j / size) : (i == j);
            if (keep) { dA[r] += tA[r]; dAn[r] += tAn[r]; dP[r] += tP[r]; }
        }
        // the next level overwrites the tiles this wave has just read
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
    // waves 4-7 hand their partial sums to waves 0-3 through the upper channel half of their own
    // block's level rows (DK bytes a row, 16 bytes per lane and sum: DK / 16 lanes a row); the
    // second barrier keeps these reads ahead of T's diagonal blocks, whose rows overlap
    {
        constexpr int LPR = DK / 16, RPS = 64 / LPR;  // lanes per row, rows per sum
        static_assert(3 * RPS <= 48, "the partial sums fit the block's level rows");
        char* hand = reinterpret_cast<char*>(lv + DK / 2) + (lane / LPR) * LDK * 2 + (lane % LPR) * 16;
        if (wave >= 4) {
            *reinterpret_cast<f32x4*>(hand) = dA;
            *reinterpret_cast<f32x4*>(hand + RPS * LDK * 2) = dAn;
            *reinterpret_cast<f32x4*>(hand + 2 * RPS * LDK * 2) = dP;
        }
        lds_barrier();
        if (wave < 4) {
            dA += *reinterpret_cast<const f32x4*>(hand);
            dAn += *reinterpret_cast<const f32x4*>(hand + RPS * LDK * 2);
            dP += *reinterpret_cast<const f32x4*>(hand + 2 * RPS * LDK * 2);
        }
        lds_barrier();
    }
    if (wave < 4) {
        float p[4];
        acc_to_array(dP, p);
        put_p(I * 16 + l16, I * 16 + g4 * 4, p);
        const f32x4 t = unit_lower_inverse(dA, dAn, l16, g4);
        store_tdiag<G>(smem, I, l16, g4, t);
        put_t(I, t);
    }
}

// The same out of line, for a loop whose register allocation the strong path must not raise.
// (Its LDS and global accesses then go through flat addresses; strong chunks are rare there.)
// (Its inputs come from global memory, where the element phase's copies are in L2.)
template <typename G, int DK, typename Gt, typename PutP, typename PutT>
__device__ __noinline__ void strong_ap(char* smem, const bf16* __restrict__ q, const bf16* __restrict__ k,
                                       const bf16* __restrict__ bgate, const typename Gt::Decay* __restrict__ decay,
                                       int64_t chunk_base, int64_t tok_stride_k, int ntok, PutP put_p,
                                       PutT put_t) {
    constexpr int CPL = DK / 32;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, I = wave & 3, hf = wave >> 2, ts = lane >> 4;
    const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
    auto src = [=](int m, float (&g)[CPL], float (&xq)[CPL], float (&xk)[CPL], float (&xb)[CPL]) {
        const int64_t off = chunk_base + (int64_t)min(I * 16 + ts * 4 + m, ntok - 1) * tok_stride_k + c0;
        const auto vg = load_vec<typename Gt::Decay, CPL>(decay + off);
        const auto vq = load_vec<bf16, CPL>(q + off);
        const auto vk = load_vec<bf16, CPL>(k + off);
        const auto vb = load_vec<bf16, CPL>(bgate + off);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            g[c] = (float)vg.v[c];
            xq[c] = (float)vq.v[c];
            xk[c] = (float)vk.v[c];
            xb[c] = (float)vb.v[c];
        }
    };
    strong_ap_body<G, DK, Gt>(smem, src, ntok, put_p, put_t);
}

}  // namespace cb
}  // namespace gdn2
