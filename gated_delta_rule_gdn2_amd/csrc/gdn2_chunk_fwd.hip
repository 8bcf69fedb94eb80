// gdn2_chunk_fwd.hip -- chunk-parallel forward of the GDN-2 recurrence on gfx950.
//
// Method (page "Why NVIDIA Gated DeltaNet-2 separates erase and write gates",
// axbrief.com, section "Gated Delta Rule-2", recurrence equation, chunk size 64):
//
//   S_t = (I - k_t (b_t.k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t.v_t)^T,  o_t = S_t^T q_t.
//
// Within a chunk of C = 64 tokens (local index i, j) write G_i = sum_{s<=i} g_s
// (g = log alpha, chunk-local, per key channel) and Gamma_{i<-j} = e^{G_i - G_j}.
// Unrolling the recurrence over the chunk gives, with S the state entering it,
//
//   A[i,j] = sum_c (b.k)_ic Gamma_{i<-j,c} k_jc  (j < i),   T = (I + A)^{-1}
//   P[i,j] = sum_c  q_ic    Gamma_{i<-j,c} k_jc  (j <= i)
//   U      = T (w.v) - W S,   W = T ((b.k).Gamma)                  (gated residuals)
//   O      = (q.Gamma) S + P U
//   S_next = Diag(Gamma_C) S + (k.Gamma')^T U,   Gamma_i = e^{G_i}, Gamma'_j = e^{G_63 - G_j}.
//
// This is the representation of a block of rank-1 updates as matrix products
// (page "Why Qwen3.5 chose Gated DeltaNet", laonpeople.com, section on the WY
// representation turning sequential updates into GEMMs); A is asymmetric
// because the erase reads with b.k but writes along k.
//
// Decay factors are never formed by dividing by a cumulative product that can
// underflow (page "Muir ...", molayo1419.me, item 3: decays pivoted at
// boundaries stay in (0, 1]).  Two variants, chosen per chunk:
//   * mild chunk (every channel's whole-chunk decay Gamma_C >= 2^-64): one pivot
//     at the chunk start; the column factor 1/Gamma_j <= 2^64 is finite, so A
//     and P are single MFMA products of (b.k.Gamma), (q.Gamma) with k/Gamma.
//   * strong chunk: the chunk is split recursively at midpoints (64, 32, 16,
//     8, 4, 2 tokens).  Every pair j < i straddles exactly one split point p,
//     and Gamma_{i<-j} = Gamma_{i<-p} Gamma_{p<-j} with both factors <= 1, so
//     each level is one masked MFMA pass whose operands never overflow; the
//     diagonal of P is a last, unscaled pass.  Nothing is clamped.
//
// Precision of the bf16 path: inputs are bf16, every product accumulates in
// fp32, the state stays fp32.  Operands that are not bf16 values themselves
// (w.v, the residuals U and the matrix P) enter the MFMAs as a hi + lo pair
// of bf16 numbers (about 16 mantissa bits); o can be written in fp32.
//
// Work decomposition: one workgroup (256 threads, 4 waves) per (sequence b,
// head h, slice of DVS value columns); the columns of S are independent, so
// slices never talk to each other.  Each workgroup walks the chunks in order,
// keeps its fp32 state slice in MFMA accumulators for the whole sequence and
// recomputes the key-side quantities (A, P, T, W) itself.
#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {

template <typename T, int DK, int DVS>
struct ChunkCfg {
    static constexpr int C = 64;
    static constexpr int NT = 256;                 // threads per workgroup
    static constexpr int CPL = DK / 16;            // key channels per lane in the element phase
    static constexpr int NCT = DVS / 16;           // 16-wide value column tiles per slice
    static constexpr bool SPLIT = sizeof(T) == 2;  // hi/lo operand pairs for the bf16 path
    static constexpr int NS = SPLIT ? 2 : 1;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int PAD = 16 / ES;
    static constexpr int LDK = DK + PAD;           // row stride of [64][DK] tiles (elements)
    static constexpr int LC = C + PAD;             // row stride of [*][64] tiles (elements)
    // persistent regions (byte offsets)
    static constexpr int QG = 0;                                    // [64][LDK] q.Gamma
    static constexpr int BGT_BYTES = (DK * LC > C * LDK ? DK * LC : C * LDK) * ES;
    static constexpr int BGT = QG + C * LDK * ES;                   // [DK][LC] (b.k.Gamma)^T, then W [64][LDK]
    static constexpr int KGT = BGT + BGT_BYTES;                     // [DK][LC] (k.Gamma')^T
    static constexpr int PM = KGT + DK * LC * ES;                   // NS x [64][LC] P (hi, lo)
    static constexpr int AOP = PM + NS * C * LC * ES;               // [64][LC] A
    static constexpr int WORK = AOP + C * LC * ES;                  // time-shared work area
    // work area, element/A-P phase: mild -> BG, KI rows; strong -> 12 groups of 16 rows
    static constexpr int W_AP = 192 * LDK * ES;
    // work area, solve phase: T and T^T as MFMA operands
    static constexpr int TOP = WORK;
    static constexpr int TOPT = TOP + C * LC * ES;
    static constexpr int W_T = 2 * C * LC * ES;
    static constexpr int WORK_BYTES = W_AP > W_T ? W_AP : W_T;
    static constexpr int WVT = WORK + WORK_BYTES;                   // NS x [DVS][LC] (w.v)^T hi, lo
    static constexpr int GC = WVT + NS * DVS * LC * ES;             // [DK] fp32 Gamma_C
    static constexpr int BLK = GC + DK * 4;                         // [4][DK] fp32 block decays
    static constexpr int BYTES = BLK + 4 * DK * 4;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(BYTES >= 4 * (kMaxSort + 1), "no room for the sequence order");
    static_assert(DK % 64 == 0 && DVS % 16 == 0 && DVS <= 64, "shape");
};

__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
    hi = (bf16)x;
    lo = (bf16)(x - (float)hi);
}

// hi / lo B-fragments from an accumulator pair (contraction rows [0,16) and [16,32))
template <typename T> struct SplitFrag { Frag<T> hi, lo; };
template <typename T> __device__ __forceinline__ SplitFrag<T> split_from_acc(const f32x4& a, const f32x4& b);
template <> __device__ __forceinline__ SplitFrag<bf16> split_from_acc<bf16>(const f32x4& a, const f32x4& b) {
    SplitFrag<bf16> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16 h, l;
        split_bf16(a[e], h, l); f.hi.v[e] = h; f.lo.v[e] = l;
        split_bf16(b[e], h, l); f.hi.v[e + 4] = h; f.lo.v[e + 4] = l;
    }
    return f;
}
template <> __device__ __forceinline__ SplitFrag<float> split_from_acc<float>(const f32x4& a, const f32x4& b) {
    SplitFrag<float> f;
    f.hi = frag_from_acc<float>(a, b);
    return f;
}

template <typename T>
__device__ __forceinline__ void store_split(T* hi, T* lo, float x);
template <> __device__ __forceinline__ void store_split<bf16>(bf16* hi, bf16* lo, float x) {
    bf16 h, l;
    split_bf16(x, h, l);
    *hi = h;
    *lo = l;
}
template <> __device__ __forceinline__ void store_split<float>(float* hi, float*, float x) { *hi = x; }

// N consecutive values converted to T and written with vector stores (p aligned to 16 bytes or to
// N * sizeof(T), whichever is smaller)
template <typename T, int N>
__device__ __forceinline__ void store_vec(T* p, const float (&x)[N]) {
    if constexpr (N == 1) {
        *p = from_f32<T>(x[0]);
    } else {
        typedef T V __attribute__((ext_vector_type(N)));
        constexpr int AL = N * (int)sizeof(T) < 16 ? N * (int)sizeof(T) : 16;
        V y;
#pragma unroll
        for (int i = 0; i < N; ++i) y[i] = from_f32<T>(x[i]);
        *reinterpret_cast<V*>(__builtin_assume_aligned(p, AL)) = y;
    }
}

// the same as a hi / lo pair for bf16 (fp32: the value itself, lo unused)
template <typename T, int N>
__device__ __forceinline__ void store_vec_split(T* hi, T* lo, const float (&x)[N]) {
    if constexpr (sizeof(T) == 2) {
        float h[N], l[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            bf16 a, b;
            split_bf16(x[i], a, b);
            h[i] = (float)a;
            l[i] = (float)b;
        }
        store_vec<T, N>(hi, h);  // exact: h and l are bf16 values
        store_vec<T, N>(lo, l);
    } else {
        store_vec<T, N>(hi, x);
    }
}

// Inputs of one chunk as one thread loads them: CPL key channels of 4 tokens, and two
// value columns of TPV tokens.
template <typename T, int CPL, int TPV>
struct ChunkIn {
    Vec<float, CPL> g[4];
    Vec<T, CPL> q[4], k[4], b[4];
    Vec<T, 2> w[TPV], v[TPV];
};

// Column position inside a transposed [channel][token] bf16 tile: 16-byte units (8 tokens) are
// XOR-swizzled by (row / 16) % 8, so that the element phase's 8-byte stores to rows 8 apart hit
// distinct LDS banks; the MFMA operand loads of 16 rows share one swizzle value.  fp32 tiles
// are not swizzled.
template <typename T>
__device__ __forceinline__ int swz(int row, int col) {
    if constexpr (sizeof(T) == 2) return (((col >> 3) ^ ((row >> 4) & 7)) << 3) | (col & 7);
    else return col;
}

// permuted-map operand from a swizzled transposed tile (the two 4-element halves separately)
template <typename T>
__device__ __forceinline__ Frag<T> load_perm_swz(const T* tile, int row, int ldc, int col) {
    const T* r = tile + row * ldc;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(r + swz<T>(row, col));
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(r + swz<T>(row, col + 16));
        f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        f = load_perm(r + col);
    }
    return f;
}

// Store a transposed 16x16 A/P block pair: lane holds entry (i = l16, j = 4*g4 + r) of block
// (Ib, Jb).  With diag = 1 the block is on the diagonal: A keeps j < i, P keeps j <= i.
template <typename T>
__device__ __forceinline__ void store_AP(T* sA, T* sPh, T* sPl, int Ib, int Jb, int l16, int g4,
                                         const f32x4& accA, const f32x4& accP, int diag) {
    constexpr int ES = (int)sizeof(T), LC = 64 + 16 / ES;
    float a[4], p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = g4 * 4 + r;
        a[r] = (!diag || j < l16) ? accA[r] : 0.f;
        p[r] = (!diag || j <= l16) ? accP[r] : 0.f;
    }
    const int pidx = (Ib * 16 + l16) * LC + Jb * 16 + g4 * 4;
    store_vec<T, 4>(sA + pidx, a);
    store_vec_split<T, 4>(sPh + pidx, sPl + pidx, p);
}

// A and P of a strong-decay chunk (some channel decays below 2^-64 over the chunk): the chunk is
// split recursively at its midpoints and every pair (i, j) is formed at the level whose split
// point p it straddles, as Gamma_{i<-p} Gamma_{p<-j} with both factors <= 1.  Levels 64 and 32
// span blocks and read the row/column groups the element phase wrote to the work area; levels 16
// to 2 lie inside one 16-token block and are formed here.  Kept out of line: it runs only for
// strong chunks and would otherwise raise the register allocation of the whole loop.
template <typename T, int DK>
__device__ __noinline__ void strong_ap(T* sWork, T* sA, T* sPh, T* sPl, const T* __restrict__ q,
                                   const T* __restrict__ k, const T* __restrict__ bgate,
                                   const float* __restrict__ log_alpha, int64_t chunk_base,
                                   int64_t tok_stride_k, int ntok) {
    constexpr int CPL = DK / 16, PAD = 16 / (int)sizeof(T), LDK = DK + PAD;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int I = wave, ts = lane >> 4, c0 = (lane & 15) * CPL;
    // ---- strong decay: level 64 (pairs (2,0) (2,1) (3,0) (3,1)) and level 32 ((1,0) (3,2)) ----
    // wave 0: (2,0) (1,0); wave 1: (2,1) (3,2); wave 2: (3,0); wave 3: (3,1)
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
        int Ib = -1, Jb = -1, ga = 0, gp = 0, gcol = 0;
        if (pi == 0) {
            Ib = wave < 2 ? 2 : 3;
            Jb = wave & 1;
            ga = Ib - 2; gp = Ib; gcol = 4 + Jb;
        } else if (wave < 2) {
            Ib = wave == 0 ? 1 : 3;
            Jb = Ib - 1;
            ga = 6 + Ib / 2; gp = 8 + Ib / 2; gcol = 10 + Jb / 2;
        }
        if (Ib >= 0) {
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int kc = kk * 32 + g4 * 8;
                Frag<T> fk = load_contig(sWork + (gcol * 16 + l16) * LDK + kc);
                Frag<T> fa = load_contig(sWork + (ga * 16 + l16) * LDK + kc);
                Frag<T> fq = load_contig(sWork + (gp * 16 + l16) * LDK + kc);
                mma(accA, fk, fa);
                mma(accP, fk, fq);
            }
            store_AP<T>(sA, sPh, sPl, Ib, Jb, l16, g4, accA, accP, 0);
        }
    }
    // ---- levels 16, 8, 4, 2 inside the diagonal block I = wave, then P's diagonal ----
    // decays of this lane's tokens, and the 4-token product of the token slot ts ^ 1
    float al[CPL][4], x16[CPL];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = I * 16 + ts * 4 + m;
        const Vec<float, CPL> g = load_vec<float, CPL>(log_alpha + chunk_base + (int64_t)min(i, ntok - 1) * tok_stride_k + c0);
#pragma unroll
        for (int c = 0; c < CPL; ++c) al[c][m] = i < ntok ? exp_neg(g.v[c]) : 1.f;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) x16[c] = __shfl_xor(al[c][0] * al[c][1] * al[c][2] * al[c][3], 16);
    __syncthreads();  // the level tiles below reuse the work area
    T* lv = sWork + (wave * 48) * LDK;  // rows: [0,16) A rows, [16,32) P rows, [32,48) columns
    f32x4 dA = zero4(), dP = zero4();
#pragma unroll
    for (int L = 0; L < 5; ++L) {
        const int size = L < 4 ? (16 >> L) : 1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = ts * 4 + m;  // token within the block
            // q, k, b of this token, reloaded per level (L2) to keep few registers live
            const bool valid = I * 16 + i < ntok;
            const int64_t off = chunk_base + (int64_t)min(I * 16 + i, ntok - 1) * tok_stride_k + c0;
            const Vec<T, CPL> xq = load_vec<T, CPL>(q + off);
            const Vec<T, CPL> xk = load_vec<T, CPL>(k + off);
            const Vec<T, CPL> xb = load_vec<T, CPL>(bgate + off);
            // split point p of the segment of i (last token of its lower half); a token in the
            // upper half is a row with factor Gamma_{i<-p}, one in the lower half a column with
            // factor Gamma_{p<-i}; both are products of at most one lane's decays and x16
            bool row = false;
            float f[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                // products over this lane's tokens up to and including m, and after m
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
                const float qv = valid ? to_f32(xq.v[c]) : 0.f;
                const float kv = valid ? to_f32(xk.v[c]) : 0.f;
                const float bk = valid ? to_f32(xb.v[c]) * kv : 0.f;
                if (L == 4) {
                    ra[c] = 0.f; rp[c] = qv; cl[c] = kv;
                } else {
                    ra[c] = row ? bk * f[c] : 0.f;
                    rp[c] = row ? qv * f[c] : 0.f;
                    cl[c] = row ? 0.f : kv * f[c];
                }
            }
            store_vec<T, CPL>(lv + i * LDK + c0, ra);
            store_vec<T, CPL>(lv + (16 + i) * LDK + c0, rp);
            store_vec<T, CPL>(lv + (32 + i) * LDK + c0, cl);
        }
        __syncthreads();
        // transposed: lane holds entry (i = l16, j = 4*g4 + r) of the block
        f32x4 tA = zero4(), tP = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const int kc = kk * 32 + g4 * 8;
            Frag<T> fk = load_contig(lv + (32 + l16) * LDK + kc);
            Frag<T> fq = load_contig(lv + (16 + l16) * LDK + kc);
            mma(tP, fk, fq);
            if (L < 4) {
                Frag<T> fa = load_contig(lv + l16 * LDK + kc);
                mma(tA, fk, fa);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = l16, j = g4 * 4 + r;
            const bool keep = L < 4 ? (i / size == j / size) : (i == j);
            if (keep) { dA[r] += tA[r]; dP[r] += tP[r]; }
        }
        __syncthreads();
    }
    store_AP<T>(sA, sPh, sPl, wave, wave, l16, g4, dA, dP, 0);
}

template <typename T, typename OutT, int DK, int DV, int DVS>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const T* __restrict__ bgate, const T* __restrict__ wgate,
    const float* initial_state, OutT* __restrict__ o, float* final_state, int B, int Tparam, int H,
    int nslices, int xcd_map, const int64_t* __restrict__ cu_seqlens) {
    using Cfg = ChunkCfg<T, DK, DVS>;
    constexpr int C = Cfg::C, CPL = Cfg::CPL, NCT = Cfg::NCT;
    constexpr int LDK = Cfg::LDK, LC = Cfg::LC;
    constexpr bool SPLIT = Cfg::SPLIT;
    constexpr int TPV = C * DVS / (2 * Cfg::NT);  // tokens per thread for w.v (two columns each)
    __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
    T* sQG = reinterpret_cast<T*>(smem + Cfg::QG);
    T* sBGT = reinterpret_cast<T*>(smem + Cfg::BGT);
    T* sW = sBGT;  // W = T (b.k.Gamma) replaces (b.k.Gamma)^T once that is consumed
    T* sKGT = reinterpret_cast<T*>(smem + Cfg::KGT);
    T* sPh = reinterpret_cast<T*>(smem + Cfg::PM);
    T* sPl = sPh + C * LC;  // only used with SPLIT
    T* sA = reinterpret_cast<T*>(smem + Cfg::AOP);
    T* sWork = reinterpret_cast<T*>(smem + Cfg::WORK);
    T* sTop = reinterpret_cast<T*>(smem + Cfg::TOP);
    T* sTopT = reinterpret_cast<T*>(smem + Cfg::TOPT);
    T* sWVh = reinterpret_cast<T*>(smem + Cfg::WVT);
    T* sWVl = sWVh + DVS * LC;  // only used with SPLIT
    float* sGC = reinterpret_cast<float*>(smem + Cfg::GC);
    float* sBLK = reinterpret_cast<float*>(smem + Cfg::BLK);

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
    const int col0 = slice * DVS;  // first value column of this slice
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


    // upper blocks of A and P are never written below: clear once
    for (int x = tid; x < C * LC; x += Cfg::NT) sA[x] = from_f32<T>(0.f);
    for (int x = tid; x < Cfg::NS * C * LC; x += Cfg::NT) sPh[x] = from_f32<T>(0.f);

    // ---- state slice in accumulators: wave w owns column tiles w, w+4, ... ----
    constexpr int TPW = NCT >= 4 ? NCT / 4 : 1;  // column tiles per owning wave
    const bool owner = (NCT >= 4) || (wave < NCT);
    f32x4 S[TPW][DK / 16];
#pragma unroll
    for (int a = 0; a < TPW; ++a)
#pragma unroll
        for (int st = 0; st < DK / 16; ++st) S[a][st] = zero4();
    if (owner && initial_state) {
#pragma unroll
        for (int a = 0; a < TPW; ++a) {
            const int ct = wave + 4 * a;
            const float* src = initial_state + ((int64_t)bh * DK) * DV + col0 + ct * 16 + l16;
#pragma unroll
            for (int st = 0; st < DK / 16; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[a][st][r] = src[(int64_t)(st * 16 + g4 * 4 + r) * DV];
        }
    }

    const int nchunks = (Tlen + C - 1) / C;
    const int64_t tok_stride_k = (int64_t)H * DK;  // elements between consecutive tokens
    const int64_t tok_stride_v = (int64_t)H * DV;
    const int64_t seq_base_k = (tok0 * H + h) * DK;
    const int64_t seq_base_v = (tok0 * H + h) * DV;
    // element phase: wave I = 16-token block I; lane = (token slot ts, channel group cg) holds
    // channels cg*CPL .. +CPL of tokens 4*ts .. 4*ts+3 of the block (one 16-byte load per token)
    const int I = wave;
    const int ts = lane >> 4;
    const int c0 = (lane & 15) * CPL;
    const int cvp = (tid % (DVS / 2)) * 2, tgv = tid / (DVS / 2);  // w.v: column pair, token group

    // Every global load of a chunk, issued without a branch: a token past the end
    // of the sequence reads the last token and is zeroed before use.  The loads come
    // in two batches (decays and queries; keys, gates and values) so that neither
    // exceeds what one wave can keep in flight.
    auto load_first = [&](int n, ChunkIn<T, CPL, TPV>& in) {
        const int t0 = n * C;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int t = min(t0 + I * 16 + ts * 4 + m, Tlen - 1);
            const int64_t off = seq_base_k + (int64_t)t * tok_stride_k + c0;
            in.g[m] = load_vec<float, CPL>(log_alpha + off);
            in.q[m] = load_vec<T, CPL>(q + off);
        }
    };
    auto load_second = [&](int n, ChunkIn<T, CPL, TPV>& in) {
        const int t0 = n * C;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int t = min(t0 + I * 16 + ts * 4 + m, Tlen - 1);
            const int64_t off = seq_base_k + (int64_t)t * tok_stride_k + c0;
            in.k[m] = load_vec<T, CPL>(k + off);
            in.b[m] = load_vec<T, CPL>(bgate + off);
        }
#pragma unroll
        for (int i = 0; i < TPV; ++i) {
            const int t = min(t0 + tgv * TPV + i, Tlen - 1);
            const int64_t off = seq_base_v + (int64_t)t * tok_stride_v + col0 + cvp;
            in.w[i] = load_vec<T, 2>(wgate + off);
            in.v[i] = load_vec<T, 2>(v + off);
        }
    };

    ChunkIn<T, CPL, TPV> in;
    if (Tlen > 0) {
        load_first(0, in);
        load_second(0, in);
    }
    __syncthreads();

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        // =============== element phase, pass 1: per-channel decays ===============
        if (t0 + C > Tlen) {
            // tokens past the end of the sequence act as the identity: no decay, no read, no write
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (t0 + I * 16 + ts * 4 + m >= Tlen) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        in.g[m].v[c] = 0.f;
                        in.q[m].v[c] = from_f32<T>(0.f);
                        in.k[m].v[c] = from_f32<T>(0.f);
                        in.b[m].v[c] = from_f32<T>(0.f);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < TPV; ++i) {
                if (t0 + tgv * TPV + i >= Tlen) {
                    in.w[i].v[0] = in.w[i].v[1] = from_f32<T>(0.f);
                    in.v[i].v[0] = in.v[i].v[1] = from_f32<T>(0.f);
                }
            }
        }
        // al: decays; lp / ls: products over this lane's tokens up to and including m / after m;
        // x16: the 4-token product of the token slot ts ^ 1 (for the strong variant)
        float al[CPL][4], pre[CPL][4], suf[CPL][4], x16[CPL];
        {
            float blkv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float lp[4], ls[4];
                float p = 1.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    al[c][m] = exp_neg(in.g[m].v[c]);
                    p *= al[c][m];
                    lp[m] = p;
                }
                float sfx = 1.f;
#pragma unroll
                for (int m = 3; m >= 0; --m) { ls[m] = sfx; sfx *= al[c][m]; }
                // products of the other token slots of the block (lanes ts ^ 1, ts ^ 2, ts ^ 3)
                const float lt = p;
                x16[c] = __shfl_xor(lt, 16);
                const float x32 = __shfl_xor(lt, 32), x48 = __shfl_xor(lt, 48);
                // slots before ts: ts & 1 -> slot ts ^ 1, ts & 2 -> slots ts ^ 2, ts ^ 3 (and after ts alike)
                const float x3248 = x32 * x48;
                const float ex = ((ts & 1) ? x16[c] : 1.f) * ((ts & 2) ? x3248 : 1.f);
                const float es = ((ts & 1) ? 1.f : x16[c]) * ((ts & 2) ? 1.f : x3248);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    pre[c][m] = ex * lp[m];  // decay from the block start through token m
                    suf[c][m] = ls[m] * es;  // decay after token m to the block end
                }
                blkv[c] = ex * lt * es;
            }
            if (ts == 0) store_vec<float, CPL>(sBLK + I * DK + c0, blkv);
        }
        // write gate times value, transposed ([column][token]), hi / lo
        {
            float x0[TPV], x1[TPV];
#pragma unroll
            for (int i = 0; i < TPV; ++i) {
                x0[i] = to_f32(in.w[i].v[0]) * to_f32(in.v[i].v[0]);
                x1[i] = to_f32(in.w[i].v[1]) * to_f32(in.v[i].v[1]);
            }
            const int idx = cvp * LC + tgv * TPV;
            store_vec_split<T, TPV>(sWVh + idx, sWVl + idx, x0);
            store_vec_split<T, TPV>(sWVh + idx + LC, sWVl + idx + LC, x1);
        }
        __syncthreads();
        float blk[CPL][4], invgc[CPL];
        int strong = 0;
        {
            Vec<float, CPL> bl[4];
#pragma unroll
            for (int K = 0; K < 4; ++K) bl[K] = load_vec<float, CPL>(sBLK + K * DK + c0);
            float gcv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
#pragma unroll
                for (int K = 0; K < 4; ++K) blk[c][K] = bl[K].v[c];
                gcv[c] = blk[c][0] * blk[c][1] * blk[c][2] * blk[c][3];
                strong |= !(gcv[c] >= 0x1p-64f);
                invgc[c] = __builtin_amdgcn_rcpf(gcv[c]);
            }
            if (I == 0 && ts == 0) store_vec<float, CPL>(sGC + c0, gcv);
        }
        strong = __syncthreads_or(strong);

        // =============== element phase, pass 2: scaled operands ===============
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
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int tl = I * 16 + ts * 4 + m;
                    float xq[CPL], xb[CPL], xki[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float kv = to_f32(in.k[m].v[c]);
                        const float gam = before[c] * pre[c][m];
                        xq[c] = to_f32(in.q[m].v[c]) * gam;
                        xb[c] = to_f32(in.b[m].v[c]) * kv * gam;
                        kgt[c][m] = kv * suf[c][m] * after[c];
                        xki[c] = kgt[c][m] * invgc[c];
                        bgt[c][m] = xb[c];
                    }
                    store_vec<T, CPL>(sQG + tl * LDK + c0, xq);
                    store_vec<T, CPL>(sWork + tl * LDK + c0, xb);          // BG
                    store_vec<T, CPL>(sWork + (64 + tl) * LDK + c0, xki);  // KI
                }
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int tl = I * 16 + ts * 4 + m;
                    // y: level-64 rows/columns (pivot token 31), z: level-32 ones (pivots 15, 47)
                    float xq[CPL], ya[CPL], yp[CPL], za[CPL], zp[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float qv = to_f32(in.q[m].v[c]);
                        const float kv = to_f32(in.k[m].v[c]);
                        const float bk = to_f32(in.b[m].v[c]) * kv;
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
                    store_vec<T, CPL>(sQG + tl * LDK + c0, xq);
                    // 16-row groups: g0,g1 A rows (blocks 2,3), g2,g3 P rows, g4,g5 columns (blocks 0,1);
                    // g6,g7 A rows (blocks 1,3), g8,g9 P rows, g10,g11 columns (blocks 0,2)
                    T* wk = sWork + (ts * 4 + m) * LDK + c0;
                    if (I >= 2) {
                        store_vec<T, CPL>(wk + (I - 2) * 16 * LDK, ya);
                        store_vec<T, CPL>(wk + I * 16 * LDK, yp);
                    } else {
                        store_vec<T, CPL>(wk + (4 + I) * 16 * LDK, ya);
                    }
                    if (I & 1) {
                        store_vec<T, CPL>(wk + (6 + I / 2) * 16 * LDK, za);
                        store_vec<T, CPL>(wk + (8 + I / 2) * 16 * LDK, zp);
                    } else {
                        store_vec<T, CPL>(wk + (10 + I / 2) * 16 * LDK, za);
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int row = c0 + c;
                store_vec<T, 4>(sBGT + row * LC + swz<T>(row, I * 16 + ts * 4), bgt[c]);
                store_vec<T, 4>(sKGT + row * LC + swz<T>(row, I * 16 + ts * 4), kgt[c]);
            }
        }
        __syncthreads();

        // decays and queries of the next chunk are loaded while this one finishes (a strong
        // chunk issues them after its A and P, which need many registers)
        const int nnext = n + 1 < nchunks ? n + 1 : n;

        // =============== A and P ===============
        if (!strong) {
            load_first(nnext, in);
            // single pivot at the chunk start: A = BG KI^T, P = QG KI^T on the lower blocks
#pragma unroll
            for (int pi = 0; pi < 3; ++pi) {
                const int p = wave + 4 * pi;
                if (p < 10) {
                    // pair list (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
                    const int Ib = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
                    const int Jb = p - (Ib * (Ib + 1)) / 2;
                    // transposed tiles: lane holds A[Ib*16 + l16][Jb*16 + 4*g4 + r], same for P
                    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        const int kc = kk * 32 + g4 * 8;
                        Frag<T> fk = load_contig(sWork + (64 + Jb * 16 + l16) * LDK + kc);
                        Frag<T> fa = load_contig(sWork + (Ib * 16 + l16) * LDK + kc);
                        Frag<T> fq = load_contig(sQG + (Ib * 16 + l16) * LDK + kc);
                        mma(accA, fk, fa);
                        mma(accP, fk, fq);
                    }
                    store_AP<T>(sA, sPh, sPl, Ib, Jb, l16, g4, accA, accP, Ib > Jb ? 0 : 1);
                }
            }
        } else {
            strong_ap<T, DK>(sWork, sA, sPh, sPl, q, k, bgate, log_alpha, seq_base_k + (int64_t)t0 * tok_stride_k,
                             tok_stride_k, Tlen - t0);
            load_first(nnext, in);
        }
        __syncthreads();

        // =============== T = (I + A)^{-1}, unit lower triangular ===============
        // diagonal 16x16 blocks by forward substitution, column j on lane j of wave I;
        // the updates of step m to rows m+1..15 are independent of each other
        if (lane < 16) {
            const int j = lane;
            const T* Ab = sA + (wave * 16) * LC + wave * 16;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                const float xm = x[m];
#pragma unroll
                for (int i = m + 1; i < 16; ++i) x[i] -= to_f32(Ab[i * LC + m]) * xm;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sTop[(wave * 16 + i) * LC + wave * 16 + j] = from_f32<T>(x[i]);
            store_vec<T, 16>(sTopT + (wave * 16 + j) * LC + wave * 16, x);
        }
        // clear T above the diagonal blocks (rows of block I, columns past block I)
        for (int x = lane; x < 16 * 64; x += 64) {
            const int i = x >> 6, cidx = x & 63;
            if (cidx >= (wave + 1) * 16) sTop[(wave * 16 + i) * LC + cidx] = from_f32<T>(0.f);
        }
        __syncthreads();
        // off-diagonal blocks by sub-diagonal: T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            if (wave < 4 - d) {
                const int Jb = wave, Ib = wave + d;
                f32x4 z = zero4();
                for (int Kb = Jb; Kb < Ib; ++Kb) {
                    const Frag16<T> fa = load16(sA + (Ib * 16 + l16) * LC + Kb * 16 + 4 * g4);
                    const Frag16<T> ft = load16(sTopT + (Jb * 16 + l16) * LC + Kb * 16 + 4 * g4);
                    mma16(z, fa, ft);
                }
                f32x4 tij = zero4();
                mma16(tij, load16(sTop + (Ib * 16 + l16) * LC + Ib * 16 + 4 * g4), frag16_from_acc<T>(z));
                float nt[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    nt[r] = -tij[r];
                    sTop[(Ib * 16 + g4 * 4 + r) * LC + Jb * 16 + l16] = from_f32<T>(nt[r]);
                }
                store_vec<T, 4>(sTopT + (Jb * 16 + l16) * LC + Ib * 16 + g4 * 4, nt);
            }
            __syncthreads();
        }

        // the next chunk's keys, gates and values
        load_second(nnext, in);

        // =============== W = T (b.k.Gamma), U0 = T (w.v) ===============
        constexpr int WCT = DK / 16 / 4;  // W column tiles per wave
        // W^T tiles: lane holds W[it*16 + l16][ct*16 + 4*g4 + r]
        f32x4 Wacc[WCT][4];
#pragma unroll
        for (int a = 0; a < WCT; ++a) {
            const int ct = wave + 4 * a;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                Wacc[a][it] = zero4();
#pragma unroll
                for (int kk = 0; kk <= it / 2; ++kk) {
                    const int kc = kk * 32 + g4 * 8;
                    Frag<T> fb = load_contig(sBGT + (ct * 16 + l16) * LC + swz<T>(ct * 16 + l16, kc));
                    Frag<T> ft = load_contig(sTop + (it * 16 + l16) * LC + kc);
                    mma(Wacc[a][it], fb, ft);
                }
            }
        }
        f32x4 U[TPW][4];
        if (owner) {
#pragma unroll
            for (int a = 0; a < TPW; ++a) {
                const int ct = wave + 4 * a;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    U[a][rt] = zero4();
#pragma unroll
                    for (int kk = 0; kk <= rt / 2; ++kk) {
                        const int kc = kk * 32 + g4 * 8;
                        Frag<T> fa = load_contig(sTop + (rt * 16 + l16) * LC + kc);
                        Frag<T> fb = load_contig(sWVh + (ct * 16 + l16) * LC + kc);
                        mma(U[a][rt], fa, fb);
                        if constexpr (SPLIT) {
                            Frag<T> fl = load_contig(sWVl + (ct * 16 + l16) * LC + kc);
                            mma(U[a][rt], fa, fl);
                        }
                    }
                }
            }
        }
        __syncthreads();  // every read of (b.k.Gamma)^T is done
#pragma unroll
        for (int a = 0; a < WCT; ++a) {
            const int ct = wave + 4 * a;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const float x[4] = {Wacc[a][it][0], Wacc[a][it][1], Wacc[a][it][2], Wacc[a][it][3]};
                store_vec<T, 4>(sW + (it * 16 + l16) * LDK + ct * 16 + g4 * 4, x);
            }
        }
        __syncthreads();

        // =============== state pass ===============
        if (owner) {
            float gc[DK / 16][4];
#pragma unroll
            for (int st = 0; st < DK / 16; ++st) {
                f32x4 x4 = *reinterpret_cast<const f32x4*>(sGC + st * 16 + g4 * 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) gc[st][r] = x4[r];
            }
#pragma unroll
            for (int a = 0; a < TPW; ++a) {
                const int ct = wave + 4 * a;
                Frag<T> sf[DK / 32];
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) sf[kk] = frag_from_acc<T>(S[a][2 * kk], S[a][2 * kk + 1]);
                f32x4 X[4], Y[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) { X[rt] = zero4(); Y[rt] = zero4(); }
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    const int kc = kk * 32 + g4 * 4;
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        Frag<T> fw = load_perm(sW + (rt * 16 + l16) * LDK + kc);
                        Frag<T> fq = load_perm(sQG + (rt * 16 + l16) * LDK + kc);
                        mma(X[rt], fw, sf[kk]);
                        mma(Y[rt], fq, sf[kk]);
                    }
                }
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) U[a][rt] -= X[rt];
                SplitFrag<T> uf[2];
                uf[0] = split_from_acc<T>(U[a][0], U[a][1]);
                uf[1] = split_from_acc<T>(U[a][2], U[a][3]);
                // O = (q.Gamma) S + P U
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                    for (int kk = 0; kk <= rt / 2; ++kk) {
                        const int pofs = (rt * 16 + l16) * LC + kk * 32 + g4 * 4;
                        Frag<T> fp = load_perm(sPh + pofs);
                        mma(Y[rt], fp, uf[kk].hi);
                        if constexpr (SPLIT) {
                            mma(Y[rt], fp, uf[kk].lo);
                            Frag<T> fpl = load_perm(sPl + pofs);
                            mma(Y[rt], fpl, uf[kk].hi);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = t0 + rt * 16 + g4 * 4 + r;
                        if (t < Tlen)
                            o[seq_base_v + (int64_t)t * tok_stride_v + col0 + ct * 16 + l16] =
                                from_f32<OutT>(Y[rt][r]);
                    }
                }
                // S <- Diag(Gamma_C) S + (k.Gamma')^T U
#pragma unroll
                for (int st = 0; st < DK / 16; ++st) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[a][st][r] *= gc[st][r];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        Frag<T> fk = load_perm_swz(sKGT, st * 16 + l16, LC, kk * 32 + g4 * 4);
                        mma(S[a][st], fk, uf[kk].hi);
                        if constexpr (SPLIT) mma(S[a][st], fk, uf[kk].lo);
                    }
                }
            }
        }
        __syncthreads();
    }

    if (owner && final_state) {
#pragma unroll
        for (int a = 0; a < TPW; ++a) {
            const int ct = wave + 4 * a;
            float* dst = final_state + ((int64_t)bh * DK) * DV + col0 + ct * 16 + l16;
#pragma unroll
            for (int st = 0; st < DK / 16; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)(st * 16 + g4 * 4 + r) * DV] = S[a][st][r];
        }
    }
}

template <typename T, typename OutT, int DK, int DV, int DVS>
static hipError_t launch_chunk(const ChunkArgs& a) {
    const int nslices = DV / DVS;
    const int64_t groups = (int64_t)a.B * a.H * nslices;
    const int xcd_map = ((int64_t)a.B * a.H) % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((chunk_fwd_kernel<T, OutT, DK, DV, DVS>), dim3((unsigned)groups), dim3(256), 0,
                       (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha,
                       (const T*)a.b, (const T*)a.w, a.initial_state, (OutT*)a.o, a.final_state, (int)a.B,
                       (int)a.T, (int)a.H, nslices, xcd_map, a.cu_seqlens);
    return hipGetLastError();
}

template <typename T, typename OutT, int D>
static hipError_t launch_dvs(const ChunkArgs& a, int dvs) {
    switch (dvs) {
        case 16: return launch_chunk<T, OutT, D, D, 16>(a);
        case 32: return launch_chunk<T, OutT, D, D, 32>(a);
        case 64: return launch_chunk<T, OutT, D, D, 64>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, int dvs) {
    if (a.dk != a.dv) return hipErrorInvalidValue;
    if (a.dtype_bf16) {
        return launch_chunk_bf16(a, dvs);
    } else if (a.dk == 64 && a.out_f32) {
        return launch_dvs<float, float, 64>(a, dvs);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn2
