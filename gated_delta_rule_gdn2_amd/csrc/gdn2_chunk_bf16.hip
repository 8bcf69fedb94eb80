// gdn2_chunk_bf16.hip -- chunk-parallel forward of the GDN-2 recurrence, bf16 inputs, gfx950.
//
// The recurrence (page "Why NVIDIA Gated DeltaNet-2 separates erase and write gates",
// axbrief.com, section "Gated Delta Rule-2"; chunk size 64 from the same section):
//
//   S_t = (I - k_t (b_t.k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t.v_t)^T,   o_t = S_t^T q_t.
//
// Per chunk of C = 64 tokens, with G_i the chunk-local cumulative log decay and
// Gamma_{i<-j} = e^{G_i - G_j} per key channel (the WY form of a block of rank-1
// updates, page "Why Qwen3.5 chose Gated DeltaNet", laonpeople.com, section on the WY
// representation):
//
//   A[i,j] = sum_c (b.k)_ic Gamma_{i<-j,c} k_jc  (j < i),     P[i,j] = the same with q_i (j <= i)
//   W  = (I + A)^{-1} ((b.k).Gamma),   U0 = (I + A)^{-1} (w.v),   U = U0 - W S
//   O  = (q.Gamma) S + P U,            S_next = Diag(Gamma_C) S + (k.Gamma')^T U.
//
// Decays are pivoted so that nothing underflows into a division (page "Muir ...",
// molayo1419.me, item 3: boundary-pivoted multiplicative decays stay in (0, 1]): a chunk
// whose whole-chunk decay stays above 2^-64 in every channel uses one pivot at the chunk
// start (k / Gamma is then finite); any other chunk splits recursively at midpoints, so
// every factor is a product of decays and <= 1.
//
// Work decomposition: one workgroup of 512 threads (8 waves, two per SIMD) per
// (sequence, head, slice of DVS value columns), walking the chunks in order.
//   * element phase: wave w takes the 16-token block I = w % 4 and channel half w / 4;
//     lane = (token slot of 4 tokens, 4 or 2 channels).
//   * A, P: waves 0-3 form the diagonal block of A in both orientations in fp32
//     accumulators and invert I + A_II at once by doubling,
//         (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8),   N strictly lower 16 x 16,
//     with hi + lo bf16 MFMA products; waves 4-6 form the off-diagonal blocks.
//   * the off-diagonal blocks of T = (I + A)^{-1} through halves of 32 tokens:
//     T = [[T_A, 0], [T_C, T_B]], T_10 = -T_11 A_10 T_00, T_32 likewise, T_C = -T_B A_BA T_A.
//   * W = T (b.k.Gamma) and U0 = T (w.v), then the state pass, as independent 16 x 16 tiles
//     spread over all eight waves; the fp32 state slice lives in MFMA accumulators (four
//     tiles per wave), and S (bf16) and U (hi / lo bf16) reach the other waves through LDS.
// Operands that are not bf16 numbers themselves (w.v through U0, U, P) enter the MFMAs as
// hi + lo bf16 pairs; every product accumulates in fp32.

#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {
namespace cb {

constexpr int C = 64;
constexpr int NT = 512;

template <int DK, int DVS>
struct Cfg {
    static constexpr int CPL = DK / 32;   // key channels per lane in the element phase
    static constexpr int KT = DK / 16;    // 16-channel tiles
    static constexpr int NCT = DVS / 16;  // 16-column value tiles of the slice
    static constexpr int UPW = 4 * NCT >= 8 ? 4 * NCT / 8 : 1;  // (row, column) tiles of U, O per wave
    static constexpr int SPW = KT * NCT >= 8 ? KT * NCT / 8 : 1;  // 16 x 16 state tiles per wave
    static constexpr int LDK = DK + 8;    // bf16 row stride of [token][channel] tiles
    static constexpr int LC = C + 8;      // bf16 row stride of [*][token] tiles
    static constexpr int LCF = C + 4;     // fp32 row stride of [column][token] tiles
    static constexpr int VC = C * DVS / NT >= 4 ? 4 : C * DVS / NT;  // value columns per lane
    static constexpr int TPV = C * DVS / (NT * VC);                  // value tokens per lane
    // LDS regions (byte offsets); lifetimes within a chunk in the comments
    static constexpr int QG = 0;                              // [64][LDK] q.Gamma: element -> state
    static constexpr int KGT = QG + C * LDK * 2;              // [DK][LC] (k.Gamma')^T: element -> state
    static constexpr int BGT_BYTES = (DK > 2 * DVS ? DK : 2 * DVS) * LC * 2;
    static constexpr int BGT = KGT + DK * LC * 2;             // [DK][LC] (b.k.Gamma)^T: element -> W;
                                                              // then 2 x [DVS][LC] U^T hi, lo
    static constexpr int WVT = BGT + BGT_BYTES;               // [DVS][LCF] fp32 (w.v)^T: element -> U0
    static constexpr int PM = WVT + DVS * LCF * 4;            // 2 x [64][LC] P hi, lo: A,P -> state
    static constexpr int AM = PM + 2 * C * LC * 2;            // [64][LC] -A_IJ (J < I), (I + A_II)^{-1}
    static constexpr int RX = AM + C * LC * 2;                // work area, 192 rows of [LDK]:
                                                              //   mild: BG rows 0-63, K/Gamma rows 64-127
                                                              //   strong: group and level tiles
                                                              //   then W rows 0-63, S^T (bf16) rows
                                                              //   64-127, T = (I + A)^{-1} rows 128-
    static constexpr int SBT = RX + C * LDK * 2;
    static constexpr int TR = RX + 2 * C * LDK * 2;           // [64][LC] T, row-major
    static constexpr int GC = RX + 192 * LDK * 2;             // [DK] fp32 whole-chunk decays
    static constexpr int BLK = GC + DK * 4;                   // [4][DK] fp32 16-token block decays
    static constexpr int FLG = BLK + 4 * DK * 4;              // [8] int: per-wave strong-decay votes
    static constexpr int TTR = FLG + 8 * 4;                   // [64][LC] T^T (blocks of T_A and T_22)
    static constexpr int BYTES = TTR + C * LC * 2;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(BYTES >= 4 * (kMaxSort + 1), "no room for the sequence order");
    static_assert(SBT + DVS * LDK * 2 <= TR, "state operand does not fit the work area");
    static_assert(TR + C * LC * 2 <= GC, "T does not fit the work area");
    static_assert(DK % 64 == 0 && DVS % 16 == 0 && DVS <= 64 && TPV >= 1, "shape");
};

// Inputs of one chunk as one thread loads them: CPL key channels of 4 tokens, and VC value
// columns of TPV tokens.
template <int CPL, int TPV, int VC>
struct In {
    Vec<float, CPL> g[4];
    Vec<bf16, CPL> q[4], k[4], b[4];
    Vec<bf16, VC> w[TPV], v[TPV];
};

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
// doubling, like the mild path.  Out of line: it runs only for strong chunks and would
// otherwise raise the register allocation of the whole loop.
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
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        store_bf16<4>(row + 16, z);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<bf16*>(smem + G::TTR + ((I * 16 + g4 * 4 + r) * LC + I * 16 + l16) * 2) = (bf16)x[r];
}

template <int DK, int DVS>
__device__ __noinline__ void strong_ap(char* smem, const bf16* __restrict__ q, const bf16* __restrict__ k,
                                       const bf16* __restrict__ bgate, const float* __restrict__ log_alpha,
                                       int64_t chunk_base, int64_t tok_stride_k, int ntok) {
    using G = Cfg<DK, DVS>;
    constexpr int CPL = DK / 32, LDK = DK + 8, LC = C + 8;
    bf16* sX = reinterpret_cast<bf16*>(smem + G::RX);
    bf16* sA = reinterpret_cast<bf16*>(smem + G::AM);
    bf16* sPh = reinterpret_cast<bf16*>(smem + G::PM);
    bf16* sPl = sPh + C * LC;
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
        store_bf16_split<4>(sPh + idx, sPl + idx, p);
    }
    // ---- levels 16, 8, 4, 2 inside block I, then P's diagonal ----
    // decays of this lane's tokens, and the 4-token product of the token slot ts ^ 1
    float al[CPL][4], x16[CPL];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = I * 16 + ts * 4 + m;
        const Vec<float, CPL> g =
            load_vec<float, CPL>(log_alpha + chunk_base + (int64_t)min(i, ntok - 1) * tok_stride_k + c0);
#pragma unroll
        for (int c = 0; c < CPL; ++c) al[c][m] = i < ntok ? exp_neg(g.v[c]) : 1.f;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) x16[c] = __shfl_xor(al[c][0] * al[c][1] * al[c][2] * al[c][3], 16);
    lds_barrier();  // the level tiles below reuse the group-tile rows
    bf16* lv = sX + (I * 48) * LDK;  // rows: [0,16) A rows, [16,32) P rows, [32,48) columns
    f32x4 dA = zero4(), dAn = zero4(), dP = zero4();
#pragma unroll
    for (int L = 0; L < 5; ++L) {
        const int size = L < 4 ? (16 >> L) : 1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = ts * 4 + m;  // token within the block
            const bool valid = I * 16 + i < ntok;
            const int64_t off = chunk_base + (int64_t)min(I * 16 + i, ntok - 1) * tok_stride_k + c0;
            const Vec<bf16, CPL> xq = load_vec<bf16, CPL>(q + off);
            const Vec<bf16, CPL> xk = load_vec<bf16, CPL>(k + off);
            const Vec<bf16, CPL> xb = load_vec<bf16, CPL>(bgate + off);
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
                const float qv = valid ? (float)xq.v[c] : 0.f;
                const float kv = valid ? (float)xk.v[c] : 0.f;
                const float bk = valid ? (float)xb.v[c] * kv : 0.f;
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
        lds_barrier();
        if (wave < 4) {
            // tA: lane holds A[l16][4 g4 + r] of the block; tAn: A[4 g4 + r][l16]; tP like tA
            f32x4 tA = zero4(), tAn = zero4(), tP = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int kc = kk * 32 + g4 * 8;
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
        }
        lds_barrier();
    }
    if (wave < 4) {
        float p[4];
        acc_to_array(dP, p);
        const int idx = (I * 16 + l16) * LC + I * 16 + g4 * 4;
        store_bf16_split<4>(sPh + idx, sPl + idx, p);
        store_tdiag<G>(smem, I, l16, g4, unit_lower_inverse(dA, dAn, l16, g4));
    }
}

template <typename OutT, int DK, int DV, int DVS>
__global__ __launch_bounds__(NT) void chunk_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ log_alpha, const bf16* __restrict__ bgate, const bf16* __restrict__ wgate,
    const float* initial_state, OutT* __restrict__ o, float* final_state, int B, int Tparam, int H,
    int nslices, int xcd_map, const int64_t* __restrict__ cu_seqlens) {
    using G = Cfg<DK, DVS>;
    constexpr int CPL = G::CPL, KT = G::KT, NCT = G::NCT, SPW = G::SPW, UPW = G::UPW;
    constexpr int LDK = G::LDK, LC = G::LC, LCF = G::LCF, VC = G::VC, TPV = G::TPV;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    // regions the strong path and a few single accesses address directly; the rest goes
    // through byte offsets (see opq)
    bf16* sPh = reinterpret_cast<bf16*>(smem + G::PM);
    bf16* sPl = sPh + C * LC;
    bf16* sA = reinterpret_cast<bf16*>(smem + G::AM);
    float* sGC = reinterpret_cast<float*>(smem + G::GC);
    float* sBLK = reinterpret_cast<float*>(smem + G::BLK);
    auto B16 = [&](int byte_off) { return reinterpret_cast<bf16*>(smem + byte_off); };
    auto F32 = [&](int byte_off) { return reinterpret_cast<float*>(smem + byte_off); };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // workgroup -> (sequence, head, slice); slices of one (b, h) share an XCD
    int bh, slice;
    {
        const int id = blockIdx.x;
        if (xcd_map) {
            const int kk = id >> 3;
            bh = 8 * (kk / nslices) + (id & 7);
            slice = kk % nslices;
        } else {
            bh = id / nslices;
            slice = id % nslices;
        }
    }
    const int h = bh % H;
    // packed sequences: the longest first
    const int bi = cu_seqlens ? longest_first(cu_seqlens, B, bh / H, Tparam, reinterpret_cast<int*>(smem)) : bh / H;
    bh = bi * H + h;
    const int col0 = slice * DVS;
    // sequence bi covers tokens [tok0, tok0 + Tlen) of the token axis: fixed length Tparam,
    // or packed sequences delimited by offsets (clamped into [0, Tparam], so any offsets
    // keep every access in range)
    int64_t tok0;
    int Tlen;
    if (cu_seqlens) {
        const int64_t lo = min(max(cu_seqlens[bi], (int64_t)0), (int64_t)Tparam);
        const int64_t hi = min(max(cu_seqlens[bi + 1], lo), (int64_t)Tparam);
        tok0 = lo;
        Tlen = (int)(hi - lo);
    } else {
        tok0 = (int64_t)bi * Tparam;
        Tlen = Tparam;
    }


    // element phase roles
    const int I = wave & 3, hf = wave >> 2;
    const int ts = lane >> 4;
    const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
    const int vcol = (tid % (DVS / VC)) * VC, vtok = (tid / (DVS / VC)) * TPV;

    // P above the diagonal blocks is never written: clear once
    for (int x = tid; x < 2 * C * LC; x += NT) sPh[x] = (bf16)0.f;

    // ---- state slice in accumulators: wave w holds the 16 x 16 tiles w + 8 i (row tile st =
    // index % KT, column tile index / KT); lane (n, g) holds S[16 st + 4 g + r][16 ct + n] ----
    f32x4 S[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) S[i] = zero4();
    if (initial_state && wave + 8 * (SPW - 1) < KT * NCT) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int st = (wave + 8 * i) % KT, ct = (wave + 8 * i) / KT;
            const float* src = initial_state + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + ct * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[i][r] = src[(int64_t)r * DV];
        }
    }
    const bool state_owner = wave + 8 * (SPW - 1) < KT * NCT;
    const bool uo_owner = wave + 8 * (UPW - 1) < 4 * NCT;

    const int nchunks = (Tlen + C - 1) / C;
    const int64_t tok_stride_k = (int64_t)H * DK;
    const int64_t tok_stride_v = (int64_t)H * DV;
    const int64_t seq_base_k = (tok0 * H + h) * DK;
    const int64_t seq_base_v = (tok0 * H + h) * DV;

    // Every global load of a chunk, issued without a branch: a token past the end of the
    // sequence reads the last token and is zeroed before use.  Two batches (decays and
    // queries; keys, gates and values), each issued well before it is needed.
    // addresses: a per-chunk base pointer (uniform) plus a per-lane offset within the chunk,
    // (token * H * D + channel) * element size, which the host keeps below 2^24 * 4 bytes
    const int rsk = H * DK, rsv = H * DV;  // elements between consecutive tokens
    // The next chunk's inputs are loaded in two batches (decays and queries; keys, gates and
    // values), issued well before they are needed.
    auto load_first = [&](int n, In<CPL, TPV, VC>& in) {
        const int t0 = n * C, last = Tlen - 1 - t0;
        const int64_t cb = seq_base_k + (int64_t)t0 * tok_stride_k;
        const float* gb = log_alpha + cb;
        const bf16* qb = q + cb;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t e = __umul24(min(I * 16 + ts * 4 + m, last), rsk) + c0;
            in.g[m] = gload<float, CPL>(gb, e * 4);
            in.q[m] = gload<bf16, CPL>(qb, e * 2);
        }
    };
    auto load_second = [&](int n, In<CPL, TPV, VC>& in) {
        const int t0 = n * C, last = Tlen - 1 - t0;
        const int64_t cb = seq_base_k + (int64_t)t0 * tok_stride_k;
        const bf16* kb = k + cb;
        const bf16* bb = bgate + cb;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t e = __umul24(min(I * 16 + ts * 4 + m, last), rsk) + c0;
            in.k[m] = gload<bf16, CPL>(kb, e * 2);
            in.b[m] = gload<bf16, CPL>(bb, e * 2);
        }
        const int64_t cv = seq_base_v + (int64_t)t0 * tok_stride_v + col0;
        const bf16* wb = wgate + cv;
        const bf16* vb = v + cv;
#pragma unroll
        for (int i = 0; i < TPV; ++i) {
            const uint32_t e = __umul24(min(vtok + i, last), rsv) + vcol;
            in.w[i] = gload<bf16, VC>(wb, e * 2);
            in.v[i] = gload<bf16, VC>(vb, e * 2);
        }
    };

    In<CPL, TPV, VC> in;
    if (Tlen > 0) {
        load_first(0, in);
        load_second(0, in);
    }
    __syncthreads();

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int nnext = n + 1 < nchunks ? n + 1 : n;
        // lane-derived indices, recomputed every chunk: values derived from them are then
        // formed where they are used instead of being kept live (or spilled) across the loop
        const int tidv = opq(tid);
        const int lane = tidv & 63;
        const int l16 = lane & 15, g4 = lane >> 4, ts = lane >> 4;
        const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
        const int vcol = (tidv % (DVS / VC)) * VC, vtok = (tidv / (DVS / VC)) * TPV;
        // =============== element phase, pass 1: decays within the block ===============
        if (t0 + C > Tlen) {
            // tokens past the end of the sequence act as the identity: no decay, no read, no write
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (t0 + I * 16 + ts * 4 + m >= Tlen) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        in.g[m].v[c] = 0.f;
                        in.q[m].v[c] = (bf16)0.f;
                        in.k[m].v[c] = (bf16)0.f;
                        in.b[m].v[c] = (bf16)0.f;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < TPV; ++i) {
                if (t0 + vtok + i >= Tlen) {
#pragma unroll
                    for (int j = 0; j < VC; ++j) {
                        in.w[i].v[j] = (bf16)0.f;
                        in.v[i].v[j] = (bf16)0.f;
                    }
                }
            }
        }
        // decay from the block start through token m = ex * lp[m]; after token m to the block
        // end = ls[m] * es (lp, ls: this lane's 4 tokens; ex, es: the block's other token slots)
        float lp[CPL][4], ls[CPL][4], ex[CPL], es[CPL];
        {
            float blkv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float al[4];
                float p = 1.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    al[m] = exp_neg(in.g[m].v[c]);
                    p *= al[m];
                    lp[c][m] = p;
                }
                float sfx = 1.f;
#pragma unroll
                for (int m = 3; m >= 0; --m) { ls[c][m] = sfx; sfx *= al[m]; }
                // products of the other token slots of the block (lanes ts ^ 1, ts ^ 2, ts ^ 3)
                const float x16 = __shfl_xor(p, 16), x32 = __shfl_xor(p, 32), x48 = __shfl_xor(p, 48);
                const float x3248 = x32 * x48;
                ex[c] = ((ts & 1) ? x16 : 1.f) * ((ts & 2) ? x3248 : 1.f);
                es[c] = ((ts & 1) ? 1.f : x16) * ((ts & 2) ? 1.f : x3248);
                blkv[c] = ex[c] * p * es[c];
            }
            // A chunk is mild when every channel's whole-chunk decay is at least 2^-64; a
            // sufficient test that needs no second exchange: every 16-token block >= 2^-16.
            bool low = false;
#pragma unroll
            for (int c = 0; c < CPL; ++c) low |= !(blkv[c] >= 0x1p-16f);
            const int vote = __any(low);
            if (lane == 0) *reinterpret_cast<int*>(smem + G::FLG + wave * 4) = vote;
            if (ts == 0) {
                typedef float V __attribute__((ext_vector_type(CPL)));
                V x;
#pragma unroll
                for (int c = 0; c < CPL; ++c) x[c] = blkv[c];
                *reinterpret_cast<V*>(sBLK + I * DK + c0) = x;
            }
        }
        // write gate times value, transposed ([column][token]) in fp32 (exact: a product of
        // two bf16 numbers)
        const int wvb = opq(G::WVT + (vcol * LCF + vtok) * 4);
#pragma unroll
        for (int j = 0; j < VC; ++j) {
            float x[TPV];
#pragma unroll
            for (int i = 0; i < TPV; ++i) x[i] = (float)in.w[i].v[j] * (float)in.v[i].v[j];
            if constexpr (TPV == 1) {
                *F32(wvb + j * LCF * 4) = x[0];
            } else {
                typedef float V __attribute__((ext_vector_type(TPV)));
                V y;
#pragma unroll
                for (int i = 0; i < TPV; ++i) y[i] = x[i];
                *reinterpret_cast<V*>(F32(wvb + j * LCF * 4)) = y;
            }
        }
        lds_barrier();

        // =============== element phase, pass 2: scaled operands ===============
        float blk[CPL][4], invgc[CPL];
        int strong;
        {
            const int4 f0 = *reinterpret_cast<const int4*>(smem + G::FLG);
            const int4 f1 = *reinterpret_cast<const int4*>(smem + G::FLG + 16);
            strong = (f0.x | f0.y | f0.z | f0.w | f1.x | f1.y | f1.z | f1.w) != 0;
            Vec<float, CPL> bl[4];
            const int blb = opq(G::BLK + c0 * 4);
#pragma unroll
            for (int K = 0; K < 4; ++K) bl[K] = load_vec<float, CPL>(F32(blb + K * DK * 4));
            float gcv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
#pragma unroll
                for (int K = 0; K < 4; ++K) blk[c][K] = bl[K].v[c];
                gcv[c] = blk[c][0] * blk[c][1] * blk[c][2] * blk[c][3];
                invgc[c] = __builtin_amdgcn_rcpf(gcv[c]);
            }
            if (I == 0 && ts == 0) {
                typedef float V __attribute__((ext_vector_type(CPL)));
                V x;
#pragma unroll
                for (int c = 0; c < CPL; ++c) x[c] = gcv[c];
                *reinterpret_cast<V*>(sGC + c0) = x;
            }
        }
        strong = __builtin_amdgcn_readfirstlane(strong);
        {
            float before[CPL], after[CPL];  // whole blocks before / after block I
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                before[c] = 1.f;
                after[c] = 1.f;
#pragma unroll
                for (int K = 0; K < 4; ++K) {
                    if (K < I) before[c] *= blk[c][K];
                    if (K > I) after[c] *= blk[c][K];
                }
            }
            float bgt[CPL][4], kgt[CPL][4];
            if (!strong) {
                // QG = q.Gamma, BG = (b.k).Gamma, KG = k.Gamma' and KI = k / Gamma = KG / Gamma_C
                const int eb = opq(((I * 16 + ts * 4) * LDK + c0) * 2);
                const int ebx = opq(eb + G::RX);
                float bex[CPL], esa[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    bex[c] = before[c] * ex[c];
                    esa[c] = es[c] * after[c];
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float xq[CPL], xb[CPL], xki[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float kv = (float)in.k[m].v[c];
                        const float gam = bex[c] * lp[c][m];
                        xq[c] = (float)in.q[m].v[c] * gam;
                        xb[c] = (float)in.b[m].v[c] * kv * gam;
                        kgt[c][m] = kv * (ls[c][m] * esa[c]);
                        xki[c] = kgt[c][m] * invgc[c];
                        bgt[c][m] = xb[c];
                    }
                    store_bf16<CPL>(B16(eb + m * LDK * 2), xq);
                    store_bf16<CPL>(B16(ebx + m * LDK * 2), xb);
                    store_bf16<CPL>(B16(ebx + (C + m) * LDK * 2), xki);
                }
            } else {
                const int eb = opq(((I * 16 + ts * 4) * LDK + c0) * 2);
                const int wkb = opq(G::RX + (ts * 4 * LDK + c0) * 2);
                float pre[CPL][4], suf[CPL][4];
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        pre[c][m] = ex[c] * lp[c][m];
                        suf[c][m] = ls[c][m] * es[c];
                    }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // y: level-64 rows/columns (pivot token 31), z: level-32 ones (pivots 15, 47)
                    float xq[CPL], ya[CPL], yp[CPL], za[CPL], zp[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float qv = (float)in.q[m].v[c];
                        const float kv = (float)in.k[m].v[c];
                        const float bk = (float)in.b[m].v[c] * kv;
                        const float gam = before[c] * pre[c][m];
                        xq[c] = qv * gam;
                        bgt[c][m] = bk * gam;
                        kgt[c][m] = kv * suf[c][m] * after[c];
                        if (I >= 2) {
                            const float f = I == 3 ? blk[c][2] * pre[c][m] : pre[c][m];
                            ya[c] = bk * f;
                            yp[c] = qv * f;
                        } else {
                            ya[c] = kv * suf[c][m] * (I == 0 ? blk[c][1] : 1.f);
                            yp[c] = 0.f;
                        }
                        if (I & 1) {
                            za[c] = bk * pre[c][m];
                            zp[c] = qv * pre[c][m];
                        } else {
                            za[c] = kv * suf[c][m];
                            zp[c] = 0.f;
                        }
                    }
                    store_bf16<CPL>(B16(eb + m * LDK * 2), xq);
                    // 16-row groups: g0,g1 A rows (blocks 2,3), g2,g3 P rows, g4,g5 columns (blocks 0,1);
                    // g6,g7 A rows (blocks 1,3), g8,g9 P rows, g10,g11 columns (blocks 0,2)
                    bf16* wk = B16(wkb + m * LDK * 2);
                    if (I >= 2) {
                        store_bf16<CPL>(wk + (I - 2) * 16 * LDK, ya);
                        store_bf16<CPL>(wk + I * 16 * LDK, yp);
                    } else {
                        store_bf16<CPL>(wk + (4 + I) * 16 * LDK, ya);
                    }
                    if (I & 1) {
                        store_bf16<CPL>(wk + (6 + I / 2) * 16 * LDK, za);
                        store_bf16<CPL>(wk + (8 + I / 2) * 16 * LDK, zp);
                    } else {
                        store_bf16<CPL>(wk + (10 + I / 2) * 16 * LDK, za);
                    }
                }
            }
            // rows c0 .. c0 + CPL - 1 lie in one 16-row group: one swizzled offset serves them all
            const int tb = opq(G::KGT + (c0 * LC + swz(c0, I * 16 + ts * 4)) * 2);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                store_bf16<4>(B16(tb + (G::BGT - G::KGT) + c * LC * 2), bgt[c]);
                store_bf16<4>(B16(tb + c * LC * 2), kgt[c]);
            }
        }
        lds_barrier();


        // =============== A, P and the diagonal blocks of T = (I + A)^{-1} ===============
        if (!strong) {
            load_first(nnext, in);
            // single pivot at the chunk start: A = BG KI^T, P = QG KI^T on the lower blocks
            if (wave < 4) {
                // diagonal block I = wave: A_II in both orientations, then its inverse
                f32x4 nt = zero4(), nn = zero4();
                const int rk = opq(((wave * 16 + l16) * LDK + g4 * 8) * 2);
                const int rkx = opq(rk + G::RX);
                Frag<bf16> fk[DK / 32], fa[DK / 32];
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    fk[kk] = load_contig(B16(rkx + C * LDK * 2 + kk * 64));
                    fa[kk] = load_contig(B16(rkx + kk * 64));
                }
                sched_fence();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    mma(nt, fk[kk], fa[kk]);  // lane holds A[l16][4 g4 + r]
                    mma(nn, fa[kk], fk[kk]);  // lane holds A[4 g4 + r][l16]
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * g4 + r;
                    nt[r] = j < l16 ? nt[r] : 0.f;
                    nn[r] = j > l16 ? nn[r] : 0.f;
                }
                store_tdiag<G>(smem, wave, l16, g4, unit_lower_inverse(nt, nn, l16, g4));
            } else if (wave == 7) {
                // the diagonal blocks of P, so that waves 0-3 go straight to their inverses
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int rk = opq(((I * 16 + l16) * LDK + g4 * 8) * 2);
                    Frag<bf16> fk[DK / 32], fq[DK / 32];
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        fk[kk] = load_contig(B16(rk + G::RX + C * LDK * 2 + kk * 64));
                        fq[kk] = load_contig(B16(rk + kk * 64));
                    }
                    sched_fence();
                    f32x4 pd = zero4();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) mma(pd, fk[kk], fq[kk]);  // P[l16][4 g4 + r]
                    float pp[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) pp[r] = 4 * g4 + r <= l16 ? pd[r] : 0.f;
                    const int idx = (I * 16 + l16) * LC + I * 16 + g4 * 4;
                    store_bf16_split<4>(sPh + idx, sPl + idx, pp);
                }
            } else {
                // off-diagonal pairs, two per wave sharing a block row or column:
                // wave 4: (1,0) (2,0); wave 5: (2,1) (3,1); wave 6: (3,0) (3,2)
                const int rl = opq((l16 * LDK + g4 * 8) * 2);
#pragma unroll
                for (int pi = 0; pi < 2; ++pi) {
                    const int Ib = wave == 4 ? 1 + pi : wave == 5 ? 2 + pi : 3;
                    const int Jb = wave == 4 ? 0 : wave == 5 ? 1 : 2 * pi;
                    f32x4 accA = zero4(), accP = zero4();
                    Frag<bf16> fk[DK / 32], fa[DK / 32], fq[DK / 32];
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        fk[kk] = load_contig(B16(rl + G::RX + (C + Jb * 16) * LDK * 2 + kk * 64));
                        fa[kk] = load_contig(B16(rl + G::RX + Ib * 16 * LDK * 2 + kk * 64));
                        fq[kk] = load_contig(B16(rl + Ib * 16 * LDK * 2 + kk * 64));
                    }
                    sched_fence();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        mma(accA, fk[kk], fa[kk]);
                        mma(accP, fk[kk], fq[kk]);
                    }
                    float a[4], pp[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) { a[r] = -accA[r]; pp[r] = accP[r]; }
                    const int idx = (Ib * 16 + l16) * LC + Jb * 16 + g4 * 4;
                    store_bf16<4>(sA + idx, a);
                    store_bf16_split<4>(sPh + idx, sPl + idx, pp);
                }
            }
        } else {
            strong_ap<DK, DVS>(smem, q, k, bgate, log_alpha, seq_base_k + (int64_t)t0 * tok_stride_k, tok_stride_k,
                               Tlen - t0);
            load_first(nnext, in);
        }
        lds_barrier();

        // =============== off-diagonal blocks of T, through halves of 32 tokens ===============
        // T = [[T_A, 0], [T_C, T_B]] with T_A = [[T_00, 0], [T_10, T_11]], T_B likewise, and
        // T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22, T_C = -T_B A_BA T_A.  The local store
        // holds -A, so every product below adds.  B operands that are columns of T come from T^T.
        if (wave < 4) {
            // block (R, J) of T_C, one per wave: Z_xJ = (-A_x0) T_0J + (-A_x1) T_1J, then
            // T_2J = T_22 Z_2J and T_3J = T_32 Z_2J + T_33 Z_3J, formed transposed so that
            // lane (i, g) holds a row: T_RJ[i][4 g + r].  T_10 (needed for J = 0) and T_32 (for
            // R = 3) come from the diagonal blocks alone; the waves that need them form them here
            // (waves 0 and 3 also store them for the W and U0 products), so no level of their own
            // and no barrier sits between the diagonal blocks and T_C.
            const int J = wave & 1, R = 2 + (wave >> 1);
            const int tb = opq((l16 * LC + g4 * 4) * 2);
            Frag16<bf16> t10, t32;
            if (J == 0) {  // T_10 = T_11 (-A_10) T_00, lane (n, g): T_10[4 g + r][n] (T^T's orientation)
                const Frag16<bf16> fa = load16(B16(G::AM + tb + (16 * LC) * 2));
                const Frag16<bf16> fj = load16(B16(G::TTR + tb));
                const Frag16<bf16> ft = load16(B16(G::TR + tb + (16 * LC + 16) * 2));
                sched_fence();
                f32x4 z = zero4(), t = zero4();
                mma16(z, fa, fj);
                mma16(t, ft, frag16_from_acc<bf16>(z));
                t10 = frag16_from_acc<bf16>(t);
                if (wave == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) *B16(G::TR + ((16 + 4 * g4 + r) * LC + l16) * 2) = t10.v[r];
                }
            }
            if (R == 3) {  // T_32 = T_33 (-A_32) T_22, lane (i, g): T_32[i][4 g + r]
                const Frag16<bf16> fa = load16(B16(G::AM + tb + (48 * LC + 32) * 2));
                const Frag16<bf16> fj = load16(B16(G::TTR + tb + (32 * LC + 32) * 2));
                const Frag16<bf16> ft = load16(B16(G::TR + tb + (48 * LC + 48) * 2));
                sched_fence();
                f32x4 z = zero4(), t = zero4();
                mma16(z, fa, fj);
                mma16(t, frag16_from_acc<bf16>(z), ft);
                t32 = frag16_from_acc<bf16>(t);
                if (wave == 3) *reinterpret_cast<bf16x4*>(B16(G::TR + tb + (48 * LC + 32) * 2)) = t32.v;
            }
            Frag16<bf16> tf[2], a2[2], a3[2];
#pragma unroll
            for (int K = 0; K < 2; ++K) {
                if (K < J) continue;
                tf[K] = (K == 1 && J == 0) ? t10 : load16(B16(G::TTR + tb + (J * 16 * LC + K * 16) * 2));
                a2[K] = load16(B16(G::AM + tb + (32 * LC + K * 16) * 2));
                a3[K] = load16(B16(G::AM + tb + (48 * LC + K * 16) * 2));
            }
            const Frag16<bf16> t22 = load16(B16(G::TR + tb + (32 * LC + 32) * 2));
            const Frag16<bf16> t33 = load16(B16(G::TR + tb + (48 * LC + 48) * 2));
            sched_fence();
            f32x4 z2 = zero4(), z3 = zero4();
#pragma unroll
            for (int K = 0; K < 2; ++K) {
                if (K < J) continue;
                mma16(z2, a2[K], tf[K]);
                if (R == 3) mma16(z3, a3[K], tf[K]);
            }
            const Frag16<bf16> z2f = frag16_from_acc<bf16>(z2);
            f32x4 t = zero4();
            if (R == 2) {
                mma16(t, z2f, t22);
            } else {
                mma16(t, z2f, t32);
                mma16(t, frag16_from_acc<bf16>(z3), t33);
            }
            float x[4];
            acc_to_array(t, x);
            store_bf16<4>(B16(G::TR + tb + (R * 16 * LC + J * 16) * 2), x);
        }
        // the next chunk's keys, gates and values
        load_second(nnext, in);

        lds_barrier();

        // =============== W = T (b.k.Gamma), U0 = T (w.v); bf16 copy of the state ===============
        {
            // W^T tiles (column tile cw of W, row tile rt): lane (i, g) holds W[16 rt + i][16 cw + 4 g + r]
            constexpr int IPW = KT * 4 / 8;
            const int tb = opq((l16 * LC + g4 * 8) * 2);
            Frag<bf16> fb[IPW][2], ft[IPW][2];
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int it = wave * IPW + i;
                const int cw = it / 4, rt = it % 4;
                const int y = (g4 ^ cw) & 7;  // swizzle of row 16 cw + l16: unit (4 kk + g4) ^ cw
                const int bb = opq(G::BGT + (cw * 16 + l16) * LC * 2);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > rt / 2) continue;
                    fb[i][kk] = load_contig(B16(bb + (((4 * kk) ^ y) << 4)));
                    ft[i][kk] = load_contig(B16(G::TR + tb + (rt * 16 * LC + kk * 32) * 2));
                }
            }
            sched_fence();
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int it = wave * IPW + i;
                const int cw = it / 4, rt = it % 4;
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > rt / 2) continue;
                    mma(acc, fb[i][kk], ft[i][kk]);
                }
                float x[4];
                acc_to_array(acc, x);
                store_bf16<4>(B16(G::RX + ((rt * 16 + l16) * LDK + cw * 16 + g4 * 4) * 2), x);
            }
        }
        f32x4 U[UPW];
        if (uo_owner) {
            // U0 tiles (rt, ct): lane (n, g) holds U0[16 rt + 4 g + r][16 ct + n]
            const int tb = opq((l16 * LC + g4 * 8) * 2);
            f32x4 wa[UPW][2], wb[UPW][2];
            Frag<bf16> ft[UPW][2];
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int u = wave + 8 * i, ct = u % NCT, rt = u / NCT;
                const int wv = opq(G::WVT + ((ct * 16 + l16) * LCF + g4 * 8) * 4);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > rt / 2) continue;
                    wa[i][kk] = *reinterpret_cast<const f32x4*>(F32(wv + kk * 128));
                    wb[i][kk] = *reinterpret_cast<const f32x4*>(F32(wv + kk * 128 + 16));
                    ft[i][kk] = load_contig(B16(G::TR + tb + (rt * 16 * LC + kk * 32) * 2));
                }
            }
            sched_fence();
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int u = wave + 8 * i, rt = u / NCT;
                U[i] = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > rt / 2) continue;
                    Frag<bf16> fh, fl;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bf16 h, l;
                        split_bf16(wa[i][kk][e], h, l); fh.v[e] = h; fl.v[e] = l;
                        split_bf16(wb[i][kk][e], h, l); fh.v[e + 4] = h; fl.v[e + 4] = l;
                    }
                    mma(U[i], ft[i][kk], fh);
                    mma(U[i], ft[i][kk], fl);
                }
            }
        }
        if (state_owner) {
            // the state as a bf16 operand, transposed: S^T[n][c]
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int st = (wave + 8 * i) % KT, ct = (wave + 8 * i) / KT;
                float x[4];
                acc_to_array(S[i], x);
                store_bf16<4>(B16(G::SBT + ((ct * 16 + l16) * LDK + st * 16 + g4 * 4) * 2), x);
            }
        }
        lds_barrier();

        // =============== state pass ===============
        // (rt, ct) tiles: X = W S, Y^T = (q.Gamma S)^T, U = U0 - X; then O^T = Y^T + (P U)^T
        // (lane (i, g) holds O[16 rt + i][16 ct + 4 g + r]); state tiles: S <- Gamma_C S + KG^T U
        f32x4 Y[UPW];
        if (uo_owner) {
            const int rw = opq((l16 * LDK + g4 * 8) * 2);
            // every tile of this wave has column tile wave % NCT
            const int ctw = wave % NCT;
            Frag<bf16> sf[DK / 32], fw[UPW][DK / 32], fq[UPW][DK / 32];
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) sf[kk] = load_contig(B16(G::SBT + rw + (ctw * 16 * LDK + kk * 32) * 2));
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int rt = (wave + 8 * i) / NCT;
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    fw[i][kk] = load_contig(B16(G::RX + rw + (rt * 16 * LDK + kk * 32) * 2));
                    fq[i][kk] = load_contig(B16(rw + (rt * 16 * LDK + kk * 32) * 2));
                }
            }
            sched_fence();
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int u = wave + 8 * i, ct = u % NCT, rt = u / NCT;
                f32x4 X = zero4();
                Y[i] = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    mma(X, fw[i][kk], sf[kk]);
                    mma(Y[i], sf[kk], fq[i][kk]);
                }
                U[i] -= X;
                float x[4];
                acc_to_array(U[i], x);
                const int idx = ((ct * 16 + l16) * LC + rt * 16 + g4 * 4) * 2;
                store_bf16_split<4>(B16(G::BGT + idx), B16(G::BGT + DVS * LC * 2 + idx), x);
            }
        }
        lds_barrier();
        if (uo_owner) {
            const int rl = opq((l16 * LC + g4 * 8) * 2);
            // every tile of this wave has column tile wave % NCT; the last tile has the most rows
            const int ctw = wave % NCT;
            constexpr int KKU = 2;
            const int kku = ((wave + 8 * (UPW - 1)) / NCT) / 2 + 1;  // U fragments the tiles use
            Frag<bf16> uh[KKU], ul[KKU], ph[UPW][2], pl[UPW][2];
#pragma unroll
            for (int kk = 0; kk < KKU; ++kk) {
                if (kk >= kku) continue;
                const int uo = G::BGT + rl + (ctw * 16 * LC + kk * 32) * 2;
                uh[kk] = load_contig(B16(uo));
                ul[kk] = load_contig(B16(uo + DVS * LC * 2));
            }
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int rt = (wave + 8 * i) / NCT;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > rt / 2) continue;
                    const int po = G::PM + rl + (rt * 16 * LC + kk * 32) * 2;
                    ph[i][kk] = load_contig(B16(po));
                    pl[i][kk] = load_contig(B16(po + C * LC * 2));
                }
            }
            sched_fence();
            const OutT* ob = o + seq_base_v + (int64_t)t0 * tok_stride_v + col0;
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int u = wave + 8 * i, ct = u % NCT, rt = u / NCT;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > rt / 2) continue;
                    mma(Y[i], uh[kk], ph[i][kk]);
                    mma(Y[i], ul[kk], ph[i][kk]);
                    mma(Y[i], uh[kk], pl[i][kk]);
                }
                if (t0 + rt * 16 + l16 < Tlen) {
                    const uint32_t e = __umul24(rt * 16 + l16, rsv) + ct * 16 + g4 * 4;
                    OutT* dst = const_cast<OutT*>(ob) + e;
                    if constexpr (sizeof(OutT) == 4) {
                        *reinterpret_cast<f32x4*>(dst) = Y[i];
                    } else {
                        float x[4];
                        acc_to_array(Y[i], x);
                        store_bf16<4>(reinterpret_cast<bf16*>(dst), x);
                    }
                }
            }
        }
        if (state_owner) {
            const int rl = opq((l16 * LC + g4 * 8) * 2);
            // every state tile of this wave has row tile wave % KT
            const int stw = wave % KT;
            const int y = (g4 ^ stw) & 7;  // swizzle of row 16 st + l16: unit (4 kk + g4) ^ st
            const int kb = opq(G::KGT + (stw * 16 + l16) * LC * 2);
            Frag<bf16> fk[2], fh[SPW][2], fl[SPW][2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) fk[kk] = load_contig(B16(kb + (((4 * kk) ^ y) << 4)));
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int ct = (wave + 8 * i) / KT;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int uo = G::BGT + rl + (ct * 16 * LC + kk * 32) * 2;
                    fh[i][kk] = load_contig(B16(uo));
                    fl[i][kk] = load_contig(B16(uo + DVS * LC * 2));
                }
            }
            sched_fence();
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int st = (wave + 8 * i) % KT;
                S[i] *= *reinterpret_cast<const f32x4*>(sGC + st * 16 + g4 * 4);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    mma(S[i], fk[kk], fh[i][kk]);
                    mma(S[i], fk[kk], fl[i][kk]);
                }
            }
        }
        // No barrier here: the next chunk's first pass writes only the votes, the block decays
        // and (w.v)^T, which nothing above reads, and the barrier after that pass keeps its
        // operand tiles behind every wave's reads of U, P and KG^T here.
    }

    if (state_owner && final_state) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int st = (wave + 8 * i) % KT, ct = (wave + 8 * i) / KT;
            float* dst = final_state + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + ct * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)r * DV] = S[i][r];
        }
    }
}

template <typename OutT, int D, int DVS>
hipError_t launch(const ChunkArgs& a) {
    const int nslices = D / DVS;
    const int64_t groups = (int64_t)a.B * a.H * nslices;
    const int xcd_map = ((int64_t)a.B * a.H) % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((chunk_bf16_kernel<OutT, D, D, DVS>), dim3((unsigned)groups), dim3(NT), 0,
                       (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       a.log_alpha, (const bf16*)a.b, (const bf16*)a.w, a.initial_state, (OutT*)a.o,
                       a.final_state, (int)a.B, (int)a.T, (int)a.H, nslices, xcd_map, a.cu_seqlens);
    return hipGetLastError();
}

template <typename OutT, int D>
hipError_t launch_dvs(const ChunkArgs& a, int dvs) {
    switch (dvs) {
        case 16: return launch<OutT, D, 16>(a);
        case 32: return launch<OutT, D, 32>(a);
        case 64: return launch<OutT, D, 64>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace cb

hipError_t launch_chunk_bf16(const ChunkArgs& a, int dvs) {
    if (a.dk != a.dv || !a.dtype_bf16) return hipErrorInvalidValue;
    if (a.dk == 128) return a.out_f32 ? cb::launch_dvs<float, 128>(a, dvs) : cb::launch_dvs<bf16, 128>(a, dvs);
    if (a.dk == 64) return a.out_f32 ? cb::launch_dvs<float, 64>(a, dvs) : cb::launch_dvs<bf16, 64>(a, dvs);
    return hipErrorInvalidValue;
}

}  // namespace gdn2
