// gdn2_chunk_split.hip -- the chunk forward in two kernels, bf16 inputs, gfx950.
//
// The recurrence (page "Why NVIDIA Gated DeltaNet-2 separates erase and write gates",
// axbrief.com, section "Gated Delta Rule-2"; chunk size 64 from the same section) in chunk
// form (the WY form of a block of rank-1 updates, page "Why Qwen3.5 chose Gated DeltaNet",
// laonpeople.com, section on the WY representation):
//
//   A[i,j] = sum_c (b.k)_ic Gamma_{i<-j,c} k_jc  (j < i),     P[i,j] = the same with q_i (j <= i)
//   T = (I + A)^{-1},   U = T (w.v - BG S),   O = QG S + P U,   S_next = Diag(Gamma_C) S + KG^T U
//
// with QG = q.Gamma, BG = (b.k).Gamma (Gamma: decay from the chunk start through the token) and
// KG = k.Gamma' (Gamma': decay after the token to the chunk end).  Everything but the last line's
// S-products depends on the chunk's own tokens only, so it is formed for every chunk at once:
//
//   * local_kernel: one workgroup per run of consecutive chunks of a (sequence, head), the next
//     chunk's inputs loaded one chunk ahead.  Per chunk it forms QG, BG, KG^T, Gamma_C, P and T
//     -- the decay pivoting, the A / P products and the triangular inverse of the fused forward
//     (gdn2_bf16_ops.h) -- and writes them as one record.
//   * state_kernel: one workgroup of four waves per (sequence, head); wave w owns dv / 4 columns
//     of the state (two 16-column tiles at d = 128) for all dk rows, in MFMA accumulators, for
//     the whole sequence, so that each operand fragment it reads from LDS serves both tiles.
//     Per chunk: R = w.v - BG S and Y = QG S (S as a hi / lo bf16 pair), U = T R, O = Y + P U,
//     S <- Gamma_C S + KG^T U (U as a hi / lo pair), all in that wave's registers; the record,
//     w and v go from global memory straight into LDS (no register staging), the next chunk's
//     parts loading while this one is computed.
//
// The host walks the chunks in batches of about a thousand chunk-heads: the local kernel for a
// batch, then the state kernel for it, so a batch's records (67 KiB per chunk-head at d = 128)
// are read back while the GPU's last-level cache still holds them.
//
// With few chains (long sequences of few heads) the state kernel's workgroups would leave most
// compute units idle.  The state update is affine in the state, S_end = A S_start + B over any
// run of chunks, so each sequence is cut into segments: one pass finds every segment's (A, B)
// by carrying the identity (no write term) and zero (with it) through the segment, a small
// kernel chains the segments' start states, and the forward proper then walks all segments
// in parallel from those starts.  Every chunk's record is kept for the two passes.
//
// Record of one chunk-head (D = dk = dv), each part row-major, the columns of every row in the
// order rec_col gives (groups of four interleaved within blocks of 32):
//   QG [64][D] bf16 | BG [64][D] bf16 | KG^T [D][64] bf16 |
//   T: rows 0-31 x cols 0-31, then rows 32-63 x cols 0-63 (bf16; blocks above the diagonal
//   blocks are zero) | P hi, P lo: the same | Gamma_C [D] fp32 | padding to a KiB.

#include "gdn2_bf16_ops.h"
#include "gdn2_launch.h"

namespace gdn2 {
namespace sp {

using cb::C;

// ------------------------------------------------------------------ record layout ----
// Two parts, each a whole number of KiB (one 16-byte load per lane of a wave): part A, the
// operands of X = BG S and Y = QG S; part B, everything after them.
template <int D>
struct Rec {
    static constexpr int QG = 0;
    static constexpr int BG = QG + C * D * 2;
    static constexpr int A_BYTES = BG + C * D * 2;
    static constexpr int KGT = A_BYTES;            // KG^T, one bf16 plane
    static constexpr int TRI = 32 * 32 + 32 * 64;  // elements of one plane of T or P
    static constexpr int T = KGT + D * C * 2;      // one bf16 plane
    static constexpr int P = T + TRI * 2;          // hi plane, then lo plane
    static constexpr int GC = P + 2 * TRI * 2;
    static constexpr int B_BYTES = (GC + D * 4 - A_BYTES + 1023) / 1024 * 1024;
    static constexpr int BYTES = A_BYTES + B_BYTES;
    static_assert(A_BYTES % 1024 == 0, "part A in whole KiB");
};

// Position of column c in a record row: inside each block of 32 columns the groups of four are
// stored in the order 0, 4, 1, 5, 2, 6, 3, 7, so that columns 4 g .. 4 g + 3 and 16 + 4 g ..
// 16 + 4 g + 3 -- the eight contraction slots one lane of an MFMA operand takes in the permuted
// slot map -- are 16 contiguous bytes.  A group of four columns (4-aligned) stays contiguous.
__device__ __forceinline__ int rec_col(int c) {
    const int g = (c >> 2) & 7;
    return (c & ~31) | ((g & 3) << 3) | ((g >> 2) << 2) | (c & 3);
}

// element (row, col) of a triangle plane: rows 0-31 hold cols 0-31, rows 32-63 cols 0-63
__device__ __forceinline__ int tri_index(int row, int col) {
    return row < 32 ? row * 32 + rec_col(col) : 1024 + (row - 32) * 64 + rec_col(col);
}

// ------------------------------------------------------------------ local kernel ----
constexpr int NT_LOCAL = 512;

// LDS layout of the local kernel (bytes), about 95 KiB at DK = 128 (one workgroup per CU either way:
// its registers allow two waves per SIMD).
// RX: 192 rows of LDK bf16 -- mild chunk: BG rows 0-63, k / Gamma rows 64-127, QG rows 128-191;
// strong chunk: the pivoted group and level tiles.  AM: -A below the diagonal blocks; TR, TTR:
// the diagonal blocks of T and their transposes (the block inverses' inputs to T_C); on a mild
// chunk they first hold the lo plane of k / Gamma for P, and the block inverses are stored after
// P.  QGL: QG's lo plane on a mild chunk (P takes both k / Gamma and QG as hi + lo pairs).  The
// block decays and strong-decay votes of the element phase share AM's bytes (a barrier separates
// the uses).
template <int DK>
struct LocalCfg {
    static constexpr int CPL = DK / 32;
    static constexpr int LDK = DK + 8;
    static constexpr int LC = C + 8;
    static constexpr int RX = 0;
    static constexpr int QGR = RX + 2 * C * LDK * 2;  // mild: QG rows inside RX
    static constexpr int AM = RX + 192 * LDK * 2;
    static constexpr int BLK = AM;                    // [4][DK] fp32 block decays (element phase)
    static constexpr int FLG = BLK + 4 * DK * 4;      // [8] int votes (element phase)
    static constexpr int TR = AM + C * LC * 2;
    static constexpr int TTR = TR + C * LC * 2;
    static constexpr int QGL = TTR + C * LC * 2;      // mild: QG lo rows, element -> P
    static constexpr int BYTES = QGL + C * LDK * 2;
    static constexpr int KIL = TR;                    // mild: k / Gamma lo rows, element -> P (T's
                                                      // diagonal blocks land there after P)
    static_assert(BYTES <= 163840, "LDS budget");
    static_assert(KIL + C * LDK * 2 <= QGL, "k / Gamma lo plane");
    static_assert(FLG + 32 <= TR, "votes inside AM");
};

template <int CPL, typename Decay>
struct InK {
    cb::Raw<Decay, CPL> g[4];
    cb::Raw<bf16, CPL> q[4], k[4], b[4];
};

// 4 consecutive values of a row into one bf16 plane of a record (rounded once)
__device__ __forceinline__ void put4(char* rec_plane, int idx, const float (&x)[4]) {
    bf16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = (bf16)x[r];
    *reinterpret_cast<bf16x4*>(rec_plane + idx * 2) = h;
}

// 4 consecutive values of a row as hi and lo bf16 planes of a record
__device__ __forceinline__ void put_split4(char* rec_plane_hi, char* rec_plane_lo, int idx, const float (&x)[4]) {
    bf16x4 h, l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        bf16 a, b;
        cb::split_bf16(x[r], a, b);
        h[r] = a;
        l[r] = b;
    }
    *reinterpret_cast<bf16x4*>(rec_plane_hi + idx * 2) = h;
    *reinterpret_cast<bf16x4*>(rec_plane_lo + idx * 2) = l;
}

template <int DK, typename Gt>
__global__ __launch_bounds__(NT_LOCAL, 2) void local_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const typename Gt::Decay* __restrict__ decay,
    const bf16* __restrict__ bgate, char* __restrict__ recs, int Tparam, int H, int c_begin, int c_end,
    int run) {
    using G = LocalCfg<DK>;
    using R = Rec<DK>;
    constexpr int CPL = G::CPL, LDK = G::LDK, LC = G::LC;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    bf16* sA = reinterpret_cast<bf16*>(smem + G::AM);
    float* sBLK = reinterpret_cast<float*>(smem + G::BLK);
    auto B16 = [&](int byte_off) { return reinterpret_cast<bf16*>(smem + byte_off); };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = c_end - c_begin;                 // chunks per head in this batch
    const int runs = (nb + run - 1) / run;
    const int bh = blockIdx.x / runs;
    const int rr = blockIdx.x % runs;
    const int cr0 = rr * run;                       // first chunk of the run, batch-relative
    const int cr1 = min(cr0 + run, nb);
    const int h = bh % H;
    const int Tlen = Tparam;
    const int64_t tok0 = (int64_t)(bh / H) * Tparam;

    const int I = wave & 3, hf = wave >> 2;         // element phase: token block, channel half
    const int64_t tok_stride_k = (int64_t)H * DK;
    const int64_t seq_base_k = (tok0 * H + h) * DK;
    const int rsk = H * DK;

    using Decay = typename Gt::Decay;
    auto load_first = [&](int n, InK<CPL, Decay>& in) {
        const int lane = tid & 63, ts = lane >> 4;
        const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
        const int t0 = n * C, last = Tlen - 1 - t0;
        const int64_t cbase = seq_base_k + (int64_t)t0 * tok_stride_k;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t e = __umul24(min(I * 16 + ts * 4 + m, last), rsk) + c0;
            in.g[m] = cb::gload_raw<Decay, CPL>(decay + cbase, e * (uint32_t)sizeof(Decay));
            in.q[m] = cb::gload_raw<bf16, CPL>(q + cbase, e * 2);
        }
    };
    auto load_second = [&](int n, InK<CPL, Decay>& in) {
        const int lane = tid & 63, ts = lane >> 4;
        const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
        const int t0 = n * C, last = Tlen - 1 - t0;
        const int64_t cbase = seq_base_k + (int64_t)t0 * tok_stride_k;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t e = __umul24(min(I * 16 + ts * 4 + m, last), rsk) + c0;
            in.k[m] = cb::gload_raw<bf16, CPL>(k + cbase, e * 2);
            in.b[m] = cb::gload_raw<bf16, CPL>(bgate + cbase, e * 2);
        }
    };

    InK<CPL, Decay> in;
    if (cr0 < cr1) {
        load_first(c_begin + cr0, in);
        load_second(c_begin + cr0, in);
    }

    for (int cr = cr0; cr < cr1; ++cr) {
        const int n = c_begin + cr;                 // chunk index in the sequence
        const int t0 = n * C;
        const int nnext = cr + 1 < cr1 ? n + 1 : n;
        char* rec = recs + ((int64_t)bh * nb + cr) * R::BYTES;
        const int tidv = cb::opq(tid);
        const int lane = tidv & 63;
        const int l16 = lane & 15, g4 = lane >> 4, ts = lane >> 4;
        const int c0 = hf * (DK / 2) + (lane & 15) * CPL;
        // =============== element phase, pass 1: decays within the block ===============
        // Tokens past the end of the sequence (their loads read the last token) act as the identity:
        // no decay and k = 0 (which zeroes their A, P-column, BG and KG entries; q, b, w, v may stay:
        // what they feed reaches only the rows of those tokens, which are never stored).  Applied
        // where alpha and k are used, so that no register of a load still in flight is written here.
        bool tok_ok[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) tok_ok[m] = t0 + I * 16 + ts * 4 + m < Tlen;
        float lp[CPL][4], ls[CPL][4], ex[CPL], es[CPL];
        {
            float blkv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float al[4];
                float p = 1.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    al[m] = tok_ok[m] ? Gt::alpha(in.g[m].f(c)) : 1.f;
                    p *= al[m];
                    lp[c][m] = p;
                }
                float sfx = 1.f;
#pragma unroll
                for (int m = 3; m >= 0; --m) { ls[c][m] = sfx; sfx *= al[m]; }
                const float x16 = __shfl_xor(p, 16), x32 = __shfl_xor(p, 32), x48 = __shfl_xor(p, 48);
                const float x3248 = x32 * x48;
                ex[c] = ((ts & 1) ? x16 : 1.f) * ((ts & 2) ? x3248 : 1.f);
                es[c] = ((ts & 1) ? 1.f : x16) * ((ts & 2) ? 1.f : x3248);
                blkv[c] = ex[c] * p * es[c];
            }
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
        cb::lds_barrier();

        // =============== element phase, pass 2: scaled operands ===============
        float blk[CPL][4], invgc[CPL];
        int strong;
        {
            const int4 f0 = *reinterpret_cast<const int4*>(smem + G::FLG);
            const int4 f1 = *reinterpret_cast<const int4*>(smem + G::FLG + 16);
            strong = (f0.x | f0.y | f0.z | f0.w | f1.x | f1.y | f1.z | f1.w) != 0;
            Vec<float, CPL> bl[4];
#pragma unroll
            for (int K = 0; K < 4; ++K) bl[K] = load_vec<float, CPL>(sBLK + K * DK + c0);
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
                *reinterpret_cast<V*>(rec + R::GC + c0 * 4) = x;
            }
        }
        strong = __builtin_amdgcn_readfirstlane(strong);
        {
            float before[CPL], after[CPL];
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
            float kgt[CPL][4];
            // record rows of this lane's tokens: QG and BG [token][DK]
            char* rq = rec + R::QG + ((I * 16 + ts * 4) * DK + rec_col(c0)) * 2;
            char* rb = rec + R::BG + ((I * 16 + ts * 4) * DK + rec_col(c0)) * 2;
            if (!strong) {
                const int eb = cb::opq(((I * 16 + ts * 4) * LDK + c0) * 2);
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
                        const float kv = tok_ok[m] ? in.k[m].f(c) : 0.f;
                        const float gam = bex[c] * lp[c][m];
                        xq[c] = in.q[m].f(c) * gam;
                        xb[c] = Gt::gate(in.b[m].f(c)) * kv * gam;
                        kgt[c][m] = kv * (ls[c][m] * esa[c]);
                        xki[c] = kgt[c][m] * invgc[c];
                    }
                    cb::store_bf16_split<CPL>(B16(G::QGR + eb + m * LDK * 2), B16(G::QGL + eb + m * LDK * 2), xq);
                    cb::store_bf16<CPL>(B16(G::RX + eb + m * LDK * 2), xb);
                    cb::store_bf16_split<CPL>(B16(G::RX + eb + (C + m) * LDK * 2), B16(G::KIL + eb + m * LDK * 2),
                                              xki);
                    cb::store_bf16<CPL>(reinterpret_cast<bf16*>(rq + m * DK * 2), xq);
                    cb::store_bf16<CPL>(reinterpret_cast<bf16*>(rb + m * DK * 2), xb);
                }
            } else {
                const int wkb = cb::opq(G::RX + (ts * 4 * LDK + c0) * 2);
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
                    float xq[CPL], xb[CPL], ya[CPL], yp[CPL], za[CPL], zp[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float qv = in.q[m].f(c);
                        const float kv = tok_ok[m] ? in.k[m].f(c) : 0.f;
                        const float bk = Gt::gate(in.b[m].f(c)) * kv;
                        const float gam = before[c] * pre[c][m];
                        xq[c] = qv * gam;
                        xb[c] = bk * gam;
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
                    cb::store_bf16<CPL>(reinterpret_cast<bf16*>(rq + m * DK * 2), xq);
                    cb::store_bf16<CPL>(reinterpret_cast<bf16*>(rb + m * DK * 2), xb);
                    bf16* wk = B16(wkb + m * LDK * 2);
                    if (I >= 2) {
                        cb::store_bf16<CPL>(wk + (I - 2) * 16 * LDK, ya);
                        cb::store_bf16<CPL>(wk + I * 16 * LDK, yp);
                    } else {
                        cb::store_bf16<CPL>(wk + (4 + I) * 16 * LDK, ya);
                    }
                    if (I & 1) {
                        cb::store_bf16<CPL>(wk + (6 + I / 2) * 16 * LDK, za);
                        cb::store_bf16<CPL>(wk + (8 + I / 2) * 16 * LDK, zp);
                    } else {
                        cb::store_bf16<CPL>(wk + (10 + I / 2) * 16 * LDK, za);
                    }
                }
            }
            // KG^T [DK][64], rounded once: this lane's 4 tokens of each of its channels
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int e = ((c0 + c) * C + rec_col(I * 16 + ts * 4)) * 2;
                cb::store_bf16<4>(reinterpret_cast<bf16*>(rec + R::KGT + e), kgt[c]);
            }
        }
        cb::lds_barrier();

        // =============== A, P and the diagonal blocks of T = (I + A)^{-1} ===============
        char* th = rec + R::T;
        char* ph = rec + R::P;
        char* pl = rec + R::P + R::TRI * 2;
        auto put_p = [=](int row, int col, const float (&p)[4]) { put_split4(ph, pl, tri_index(row, col), p); };
        f32x4 tdiag = zero4();  // mild: waves 0-3's block inverse, stored once P is formed
        if (!strong) {
            load_first(nnext, in);
            if (wave < 4) {
                // diagonal block I = wave: A_II in both orientations, then its inverse
                f32x4 nt = zero4(), nn = zero4();
                const int rk = cb::opq(((wave * 16 + l16) * LDK + g4 * 8) * 2);
                const int rkx = cb::opq(rk + G::RX);
                Frag<bf16> fk[DK / 32], fa[DK / 32];
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    fk[kk] = load_contig(B16(rkx + C * LDK * 2 + kk * 64));
                    fa[kk] = load_contig(B16(rkx + kk * 64));
                }
                cb::sched_fence();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    mma(nt, fk[kk], fa[kk]);
                    mma(nn, fa[kk], fk[kk]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * g4 + r;
                    nt[r] = j < l16 ? nt[r] : 0.f;
                    nn[r] = j > l16 ? nn[r] : 0.f;
                }
                tdiag = cb::unit_lower_inverse(nt, nn, l16, g4);
                float x[4];
                cb::acc_to_array(tdiag, x);
                put4(th, tri_index(wave * 16 + l16, wave * 16 + g4 * 4), x);
            } else if (wave == 7) {
#pragma unroll
                for (int Ib = 0; Ib < 4; ++Ib) {
                    const int rk = cb::opq(((Ib * 16 + l16) * LDK + g4 * 8) * 2);
                    Frag<bf16> fk[DK / 32], fl[DK / 32], fq[DK / 32], fm[DK / 32];
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        fk[kk] = load_contig(B16(rk + G::RX + C * LDK * 2 + kk * 64));
                        fq[kk] = load_contig(B16(rk + G::QGR + kk * 64));
                        fl[kk] = load_contig(B16(rk + G::KIL + kk * 64));  // k / Gamma lo
                        fm[kk] = load_contig(B16(rk + G::QGL + kk * 64));  // QG lo
                    }
                    cb::sched_fence();
                    f32x4 pd = zero4();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        mma(pd, fk[kk], fq[kk]);
                        mma(pd, fl[kk], fq[kk]);
                        mma(pd, fk[kk], fm[kk]);
                    }
                    float pp[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) pp[r] = 4 * g4 + r <= l16 ? pd[r] : 0.f;
                    put_p(Ib * 16 + l16, Ib * 16 + g4 * 4, pp);
                }
            } else {
                // off-diagonal pairs: wave 4: (1,0) (2,0); wave 5: (2,1) (3,1); wave 6: (3,0) (3,2)
                const int rl = cb::opq((l16 * LDK + g4 * 8) * 2);
#pragma unroll
                for (int pi = 0; pi < 2; ++pi) {
                    const int Ib = wave == 4 ? 1 + pi : wave == 5 ? 2 + pi : 3;
                    const int Jb = wave == 4 ? 0 : wave == 5 ? 1 : 2 * pi;
                    f32x4 accA = zero4(), accP = zero4();
                    Frag<bf16> fk[DK / 32], fl[DK / 32], fa[DK / 32], fq[DK / 32];
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        fk[kk] = load_contig(B16(rl + G::RX + (C + Jb * 16) * LDK * 2 + kk * 64));
                        fa[kk] = load_contig(B16(rl + G::RX + Ib * 16 * LDK * 2 + kk * 64));
                        fq[kk] = load_contig(B16(rl + G::QGR + Ib * 16 * LDK * 2 + kk * 64));
                        fl[kk] = load_contig(B16(rl + G::KIL + Jb * 16 * LDK * 2 + kk * 64));  // k / Gamma lo
                    }
                    cb::sched_fence();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        mma(accA, fk[kk], fa[kk]);
                        mma(accP, fk[kk], fq[kk]);
                        mma(accP, fl[kk], fq[kk]);
                    }
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk)
                        fq[kk] = load_contig(B16(rl + G::QGL + Ib * 16 * LDK * 2 + kk * 64));  // QG lo
                    cb::sched_fence();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) mma(accP, fk[kk], fq[kk]);
                    float a[4], pp[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) { a[r] = -accA[r]; pp[r] = accP[r]; }
                    cb::store_bf16<4>(sA + (Ib * 16 + l16) * LC + Jb * 16 + g4 * 4, a);
                    put_p(Ib * 16 + l16, Jb * 16 + g4 * 4, pp);
                }
            }
        } else {
            // the chunk's inputs, still in the registers the element phase loaded them into (zero,
            // and no decay, past the end of the sequence)
            auto src = [&](int m, float (&g)[CPL], float (&xq)[CPL], float (&xk)[CPL], float (&xb)[CPL]) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    g[c] = in.g[m].f(c);
                    xq[c] = in.q[m].f(c);
                    xk[c] = in.k[m].f(c);
                    xb[c] = in.b[m].f(c);
                }
            };
            cb::strong_ap_body<G, DK, Gt>(smem, src, Tlen - t0, put_p, [=](int Ib, const f32x4& t) {
                                     float x[4];
                                     cb::acc_to_array(t, x);
                                     put4(th, tri_index(Ib * 16 + l16, Ib * 16 + g4 * 4), x);
                                 });
            load_first(nnext, in);
        }
        cb::lds_barrier();
        if (!strong) {
            // the k / Gamma lo rows are read: the block inverses take their place
            if (wave < 4) cb::store_tdiag<G>(smem, wave, l16, g4, tdiag);
            cb::lds_barrier();
        }

        // =============== off-diagonal blocks of T, through halves of 32 tokens ===============
        if (wave < 4) {
            const int J = wave & 1, Rb = 2 + (wave >> 1);
            const int tb = cb::opq((l16 * LC + g4 * 4) * 2);
            Frag16<bf16> t10, t32;
            if (J == 0) {  // T_10 = T_11 (-A_10) T_00, lane (n, g): T_10[4 g + r][n]
                const Frag16<bf16> fa = load16(B16(G::AM + tb + (16 * LC) * 2));
                const Frag16<bf16> fj = load16(B16(G::TTR + tb));
                const Frag16<bf16> ft = load16(B16(G::TR + tb + (16 * LC + 16) * 2));
                cb::sched_fence();
                f32x4 z = zero4(), t = zero4();
                mma16(z, fa, fj);
                mma16(t, ft, frag16_from_acc<bf16>(z));
                t10 = frag16_from_acc<bf16>(t);
                if (wave == 0) {
                    // record: T[16 + 4 g + r][n]
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<bf16*>(th + tri_index(16 + 4 * g4 + r, l16) * 2) = (bf16)t[r];
                }
            }
            if (Rb == 3) {  // T_32 = T_33 (-A_32) T_22, lane (i, g): T_32[i][4 g + r]
                const Frag16<bf16> fa = load16(B16(G::AM + tb + (48 * LC + 32) * 2));
                const Frag16<bf16> fj = load16(B16(G::TTR + tb + (32 * LC + 32) * 2));
                const Frag16<bf16> ft = load16(B16(G::TR + tb + (48 * LC + 48) * 2));
                cb::sched_fence();
                f32x4 z = zero4(), t = zero4();
                mma16(z, fa, fj);
                mma16(t, frag16_from_acc<bf16>(z), ft);
                t32 = frag16_from_acc<bf16>(t);
                if (wave == 3) {
                    float x[4];
                    cb::acc_to_array(t, x);
                    put4(th, tri_index(48 + l16, 32 + g4 * 4), x);
                }
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
            cb::sched_fence();
            f32x4 z2 = zero4(), z3 = zero4();
#pragma unroll
            for (int K = 0; K < 2; ++K) {
                if (K < J) continue;
                mma16(z2, a2[K], tf[K]);
                if (Rb == 3) mma16(z3, a3[K], tf[K]);
            }
            const Frag16<bf16> z2f = frag16_from_acc<bf16>(z2);
            f32x4 t = zero4();
            if (Rb == 2) {
                mma16(t, z2f, t22);
            } else {
                mma16(t, z2f, t32);
                mma16(t, frag16_from_acc<bf16>(z3), t33);
            }
            float x[4];
            cb::acc_to_array(t, x);
            put4(th, tri_index(Rb * 16 + l16, J * 16 + g4 * 4), x);
        } else {
            // waves 4-7: the zero blocks (0,1) and (2,3) of T and P
            const int w4 = wave - 4;                   // 0..3
            const int blkrow = w4 < 2 ? 0 : 2;         // zero blocks start at rows 0 and 32
            const float z[4] = {0.f, 0.f, 0.f, 0.f};
            const int row = blkrow * 16 + l16, col = (blkrow + 1) * 16 + g4 * 4;
            if (w4 & 1) put_split4(ph, pl, tri_index(row, col), z);
            else put4(th, tri_index(row, col), z);
        }
        // the next chunk's keys and gates
        load_second(nnext, in);
        cb::lds_barrier();
    }
}

// ------------------------------------------------------------------ state kernel ----
constexpr int NT_STATE = 256;

// XOR swizzle of 16-byte units inside a row of rb bytes (rb a power of two, 64..256), so that
// the 16 rows a fragment load touches fall on distinct LDS banks.  An involution: the same call
// maps a staged unit back to its record unit.
__device__ __forceinline__ int swz_unit(int row, int unit, int rb) {
    return unit ^ ((row * rb / 256) % (rb / 16));
}

// LDS of the state kernel.  Region A (single: its next contents load once every wave is past X,
// Y and R): part A of the record (QG, BG), then w and v of the workgroup's WGC value columns
// ([64 tokens][WGC columns] bf16 each).  Then two buffers for part B of the record (the next
// chunk's copy loads during this chunk).  A workgroup covers all D value columns: each of its
// four waves owns CT = D / 64 tiles of 16 columns, so that every operand fragment read from LDS
// feeds CT products.
template <int D>
struct StateCfg {
    using R = Rec<D>;
    static constexpr int CT = D / 64;                 // 16-column tiles per wave
    static constexpr int WGC = 64 * CT;               // value columns per workgroup
    static constexpr int WRB = WGC * 2;               // bytes of one token's w (or v) row
    static constexpr int A = 0;
    static constexpr int WV = R::A_BYTES;             // w, then v: C * WRB bytes each
    static constexpr int A_BYTES = R::A_BYTES + 2 * C * WRB;
    static constexpr int B0 = A_BYTES;
    static constexpr int BYTES = A_BYTES + 2 * R::B_BYTES;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(WGC == D, "a workgroup covers every value column");
};

// Record unit staged at LDS unit u of part A (QG then BG, rows of 2 D bytes, each swizzled).
template <int D>
__device__ __forceinline__ int src_unit_a(int u) {
    constexpr int UPR = D * 2 / 16;  // units per row
    const int row = u / UPR, un = u % UPR;
    return row * UPR + swz_unit(row, un, D * 2);
}
// The same for part B: KG^T (rows of 64 tokens, 128 bytes), the three triangle planes
// T, P hi, P lo (rows 0-31 of 64 bytes, rows 32-63 of 128 bytes), then Gamma_C and padding as
// they are.
template <int D>
__device__ __forceinline__ int src_unit_b(int u) {
    using R = Rec<D>;
    constexpr int UK = D * C * 2 / 16;          // units of the KG^T plane
    constexpr int UT = 3 * R::TRI * 2 / 16;     // units of the three triangle planes
    if (u < UK) {
        const int row = u / 8, un = u % 8;
        return row * 8 + swz_unit(row, un, 128);
    }
    if (u < UK + UT) {
        const int v = u - UK;
        constexpr int UP = R::TRI * 2 / 16;     // units of one plane: 128 (rows 0-31) + 256
        const int plane = v / UP, w = v % UP;
        const bool top = w < 128;
        const int row = top ? w / 4 : (w - 128) / 8, un = top ? w % 4 : (w - 128) % 8;
        const int sw = top ? row * 4 + swz_unit(row, un, 64) : 128 + row * 8 + swz_unit(row, un, 128);
        return UK + plane * UP + sw;
    }
    return u;
}
// w and v tiles: token t's WGC columns are a row of WRB bytes; its 16-byte units are permuted by
// XOR with 2 ((t / 4) % 4), so that the four token rows one read of the accumulator layout
// touches (4 apart, each 32 bytes of one column tile) fall on distinct banks.
__device__ __forceinline__ int wv_unit(int t, int u) { return u ^ (((t >> 2) & 3) << 1); }

typedef __attribute__((address_space(3))) void lds_void;

// One part of a record straight from global memory into LDS: load jj of the part (1 KiB) goes
// to LDS bytes [1024 jj, 1024 jj + 1024) of the part, lane l writing 16 bytes at 16 l; wave w
// takes loads jj = w, w + 4, ...  The lane's source byte offsets (the same for every record)
// come precomputed in off[].  Complete once the issuing wave's vmcnt has drained.
template <int NLOADS>
struct StageOffsets {
    static constexpr int PER_WAVE = (NLOADS + 3) / 4;
    int off[PER_WAVE];
    template <typename Src>
    __device__ __forceinline__ void init(int wave, int lane, Src src) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) off[j] = src(min(j * 4 + wave, NLOADS - 1) * 64 + lane) * 16;
    }
    // loads [SKIP_LO, SKIP_HI) are left out (parts a pass does not read)
    template <int SKIP_LO = 0, int SKIP_HI = 0>
    __device__ __forceinline__ void issue(const char* rec_part, char* lds_part, int wave) const {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int jj = j * 4 + wave;
            if (jj < NLOADS && !(jj >= SKIP_LO && jj < SKIP_HI))
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(rec_part + off[j]),
                                                 (lds_void*)(lds_part + jj * 1024), 16, 0, 0);
        }
    }
};

// A-operand fragment (permuted slot map) of row `row`, columns 32 kk .. 32 kk + 31 of a staged
// row-major part with rb-byte rows: lane (m, g) takes columns 32 kk + 4 g + e and 32 kk + 16 +
// 4 g + e (e = 0..3), the slots where a pair of accumulator tiles keeps its rows -- in the
// record's column order the 16 bytes of unit 4 kk + g, one LDS read.
__device__ __forceinline__ Frag<bf16> frag_perm(const char* part, int row, int kk, int g, int rb) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(part + row * rb + swz_unit(row, 4 * kk + g, rb) * 16);
    return f;
}

// the same from a staged triangle plane (rows 0-31: 64-byte rows; rows 32-63: 128-byte rows)
__device__ __forceinline__ Frag<bf16> frag_tri(const char* plane, int row, int kk, int g) {
    return row < 32 ? frag_perm(plane, row, kk, g, 64) : frag_perm(plane + 2048, row - 32, kk, g, 128);
}

// hi / lo K = 32 operands of an accumulator pair (permuted slot map)
__device__ __forceinline__ cb::Split32 split_pair(const f32x4& a, const f32x4& b) { return cb::split32(a, b); }

// Four waves per (sequence, head); wave w owns the 16-column tiles CT w .. CT w + CT - 1 of the
// state for all D rows, in MFMA accumulators, for the whole run of chunks; every fragment a wave
// reads serves its CT tiles.  Per chunk, two LDS-only barriers:
//   start: part B of the next record starts loading into the other B buffer;
//   X = BG S, Y = QG S (S as hi / lo), R = w.v - X, then barrier M: region A is free and the next
//   chunk's part A, w and v start loading;
//   U = T R (R as hi / lo), S <- Gamma_C S + KG^T U (U as hi / lo), O = Y + P U (P as hi / lo);
//   the wave's own loads drain, barrier F publishes the next chunk's data; O is stored after F.
// Every global access but the O stores goes straight to LDS, so a wave keeps few vector-memory
// instructions in flight.
//
// Segments (few chains: the sequence is cut into nseg runs of seg_len chunks, walked in
// parallel).  Workgroup id -> (chain, slice) with chain = segment * BH + bh.  MODE kOut: the
// forward proper; segment 0 starts from state_in, or with segments from starts[0] (a copy of it,
// so that a final state written over the initial one cannot race its read), segment g > 0 from
// starts[g]; the last
// segment writes state_out.  MODE kTrans: a segment's transition S_end = A S_start + B_seg,
// found by carrying 2 D columns through the same chunks: slices 0 .. nslices - 1 start from the
// identity and take no write term (their end state is A), slices nslices .. 2 nslices - 1 start
// from zero with the write term (B_seg); no output; the end state goes to trans[segment][bh] as
// [D][2 D] fp32.
constexpr int kOut = 0, kTrans = 1;
template <typename OutT, int D, typename Gt, int MODE>
__global__ __launch_bounds__(NT_STATE, 1) void state_kernel(
    const char* __restrict__ recs, const bf16* __restrict__ v, const bf16* __restrict__ wgate,
    const float* state_in, float* state_out, OutT* __restrict__ o, int Tparam, int H, int nslices,
    int xcd_map, int c_begin, int c_end, int BH, int seg_len, const float* __restrict__ starts,
    float* __restrict__ trans) {
    using Cf = StateCfg<D>;
    using R = Rec<D>;
    constexpr int KT = D / 16;           // 16-row key tiles of the state
    constexpr int KK = KT / 2;           // 32-row steps over the keys
    constexpr int CT = Cf::CT, WGC = Cf::WGC, WRB = Cf::WRB;
    constexpr int NLA = R::A_BYTES / 1024, NLB = R::B_BYTES / 1024;
    __shared__ __attribute__((aligned(1024))) char smem[Cf::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ns = MODE == kTrans ? 2 * nslices : nslices;  // workgroups per chain
    int chain, slice;
    {
        const int id = blockIdx.x;
        if (xcd_map) {
            const int kk = id >> 3;
            chain = 8 * (kk / ns) + (id & 7);
            slice = kk % ns;
        } else {
            chain = id / ns;
            slice = id % ns;
        }
    }
    const int seg = chain / BH, bh = chain % BH;
    const int h = bh % H;
    const int nb_all = c_end - c_begin;             // records per head
    const int s0 = seg * seg_len, nb = min(seg_len, nb_all - s0);  // this workgroup's chunks
    const int Tlen = Tparam;
    const int64_t tok0 = (int64_t)(bh / H) * Tparam;
    // the identity-start columns of a transition take no write term (w, v are staged for the
    // value slice of the same index all the same, and unused)
    const bool homog = MODE == kTrans && slice < nslices;
    const int vslice = slice < nslices ? slice : slice - nslices;
    // this lane's state / value column in tile c of the wave
    auto colc = [&](int c) { return vslice * WGC + (wave * CT + c) * 16 + l16; };
    const int64_t tok_stride_v = (int64_t)H * D;
    const char* rec0 = recs + ((int64_t)bh * nb_all + s0) * R::BYTES;
    StageOffsets<NLA> soa;
    StageOffsets<NLB> sob;
    soa.init(wave, lane, [](int u) { return src_unit_a<D>(u); });
    sob.init(wave, lane, [](int u) { return src_unit_b<D>(u); });
    // w and v of chunk n into region A: 16 CT loads of 1 KiB (TPL tokens x WGC columns of one
    // tensor), wave w taking loads w, w + 4, ...; lane l takes token TPL part + l / UPR, LDS unit
    // l % UPR of its row (swizzled: the source unit is wv_unit of it).  Tokens past the end of the
    // sequence read its last token (zeroed in R).
    constexpr int UPR = WRB / 16, TPL = 1024 / WRB, LPT = C / TPL;  // units per row, tokens and loads per tensor
    const int wv_t = lane / UPR, wv_u = lane % UPR;
    auto stage_wv = [&](int n) {
        const int t0 = n * C;
        const int last = min(C, Tlen - t0) - 1;
        const int64_t chunk = (tok0 + t0) * tok_stride_v + (int64_t)h * D + vslice * WGC;
#pragma unroll
        for (int j = 0; j < 2 * LPT / 4; ++j) {
            const int jj = j * 4 + wave, tensor = jj / LPT, part = jj % LPT;
            const int t = part * TPL + wv_t;
            const bf16* src = (tensor ? v : wgate) + chunk + (int64_t)min(t, last) * tok_stride_v + wv_unit(t, wv_u) * 8;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                             (lds_void*)(smem + Cf::WV + jj * 1024), 16, 0, 0);
        }
    };
    // A transition reads neither QG nor P (no output), and its identity-start columns no w, v
    constexpr int P_LO = (R::P - R::A_BYTES) / 1024, P_HI = (R::GC - R::A_BYTES) / 1024;
    static_assert((R::P - R::A_BYTES) % 1024 == 0 && (R::GC - R::A_BYTES) % 1024 == 0 && R::BG % 1024 == 0,
                  "parts skipped by a transition lie in whole KiB");
    auto stage_a = [&](int i) {
        if constexpr (MODE == kTrans)
            soa.template issue<0, R::BG / 1024>(rec0 + (int64_t)i * R::BYTES, smem + Cf::A, wave);
        else
            soa.issue(rec0 + (int64_t)i * R::BYTES, smem + Cf::A, wave);
        if (!homog) stage_wv(c_begin + s0 + i);
    };
    auto stage_b = [&](int i) {
        char* dst = smem + Cf::B0 + (i & 1) * R::B_BYTES;
        if constexpr (MODE == kTrans)
            sob.template issue<P_LO, P_HI>(rec0 + (int64_t)i * R::BYTES + R::A_BYTES, dst, wave);
        else
            sob.issue(rec0 + (int64_t)i * R::BYTES + R::A_BYTES, dst, wave);
    };

    // the state's CT x 16 columns of this wave, all D rows: tile (c, st), lane (n, g) holds
    // S[16 st + 4 g + r][colc(c)]
    f32x4 S[CT][KT];
    {
        const float* sin = starts ? starts + (int64_t)seg * BH * D * D : state_in;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int st = 0; st < KT; ++st) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = st * 16 + g4 * 4 + r;
                    if constexpr (MODE == kTrans)
                        S[c][st][r] = homog && row == colc(c) ? 1.f : 0.f;
                    else
                        S[c][st][r] = sin ? sin[((int64_t)bh * D + row) * D + colc(c)] : 0.f;
                }
            }
    }

    // O of a chunk through a buffer resource: the chunk's first element of this head as a uniform
    // base, the rows of its tokens as the range (a last partial chunk drops its stores past the
    // end of the sequence), this lane's column and token group as a 32-bit offset and each (tile,
    // row) step as a scalar offset -- no per-store vector address arithmetic.  Lane (n, g) of
    // tile rt holds token 16 rt + 4 g + r.
    auto store_o = [&](int n, const f32x4 (&Y)[CT][4]) {
        const int t0 = n * C;
        const int ntok = min(C, Tlen - t0);
        const auto ro = __builtin_amdgcn_make_buffer_rsrc(o + (tok0 + t0) * tok_stride_v + (int64_t)h * D, 0,
                                                          ntok * (int)tok_stride_v * (int)sizeof(OutT), 0x00020000);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const uint32_t lane_tok = (uint32_t)(g4 * 4 * tok_stride_v + colc(c));  // elements
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int so = (rt * 16 + r) * (int)tok_stride_v * (int)sizeof(OutT);
                    if constexpr (sizeof(OutT) == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, (float)Y[c][rt][r]), ro,
                                                              lane_tok * 4, so, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, from_f32<bf16>(Y[c][rt][r])),
                                                              ro, lane_tok * 2, so, 0);
                }
        }
    };

    if (nb > 0) {
        stage_a(0);
        stage_b(0);
    }
    __syncthreads();  // vmcnt(0): this wave's loads have landed; the barrier publishes every wave's

    const char* ra = smem + Cf::A;
    f32x4 Y[CT][4];
    for (int i = 0; i < nb; ++i) {
        const int n = c_begin + s0 + i;
        const int t0 = n * C;
        const char* rb = smem + Cf::B0 + (i & 1) * R::B_BYTES;
        const char* th = rb + (R::T - R::A_BYTES);
        const char* ph = rb + (R::P - R::A_BYTES);
        const char* pl = ph + R::TRI * 2;
        // part B of the next record into the other buffer (last read in the previous chunk)
        if (i + 1 < nb) stage_b(i + 1);
        // ---- X = BG S and Y = QG S, S as hi / lo bf16 pairs over 32 key rows; the fragments of
        // each step are loaded one step ahead and serve every tile of the wave ----
        f32x4 X[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) { X[c][rt] = zero4(); Y[c][rt] = zero4(); }
        Frag<bf16> fb[2][4], fq[2][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            fb[0][rt] = frag_perm(ra + R::BG, rt * 16 + l16, 0, g4, D * 2);
            if constexpr (MODE == kOut) fq[0][rt] = frag_perm(ra + R::QG, rt * 16 + l16, 0, g4, D * 2);
        }
        // the triangle fragments of U = T R: (rt, kk) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
        Frag<bf16> ft[6];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + 1 < KK) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    fb[(kk + 1) & 1][rt] = frag_perm(ra + R::BG, rt * 16 + l16, kk + 1, g4, D * 2);
                    if constexpr (MODE == kOut)
                        fq[(kk + 1) & 1][rt] = frag_perm(ra + R::QG, rt * 16 + l16, kk + 1, g4, D * 2);
                }
            } else {
#pragma unroll
                for (int p = 0; p < 6; ++p) {
                    const int rt = p < 2 ? p : 2 + (p - 2) / 2, k2 = p < 2 ? 0 : (p - 2) % 2;
                    ft[p] = frag_tri(th, rt * 16 + l16, k2, g4);
                }
            }
            // the hi products of the step for every tile, then the lo ones
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const cb::Split32 sp = split_pair(S[c][2 * kk], S[c][2 * kk + 1]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    mma(X[c][rt], fb[kk & 1][rt], sp.hi);
                    if constexpr (MODE == kOut) mma(Y[c][rt], fq[kk & 1][rt], sp.hi);
                }
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    mma(X[c][rt], fb[kk & 1][rt], sp.lo);
                    if constexpr (MODE == kOut) mma(Y[c][rt], fq[kk & 1][rt], sp.lo);
                }
            }
        }
        // ---- R = w.v - X from the staged w and v (tokens past the end of the sequence: zero) ----
        f32x4 Rr[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            // this lane's column within the w / v rows: unit and byte offset
            const int wcol = (wave * CT + c) * 16 + l16, wu = wcol >> 3, wb = (wcol & 7) * 2;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = rt * 16 + g4 * 4 + r;
                    const int off = t * WRB + wv_unit(t, wu) * 16 + wb;
                    const float wt = (float)*reinterpret_cast<const bf16*>(smem + Cf::WV + off);
                    const float vt = (float)*reinterpret_cast<const bf16*>(smem + Cf::WV + C * WRB + off);
                    Rr[c][rt][r] = (homog ? 0.f : Gt::gate(wt) * vt) - X[c][rt][r];
                }
        }
        if (t0 + C > Tlen) {
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (t0 + rt * 16 + g4 * 4 + r >= Tlen) Rr[c][rt][r] = 0.f;
        }
        // barrier M: every wave is past region A; the next chunk's part A, w and v load during the
        // rest of the chunk
        cb::lds_barrier();
        if (i + 1 < nb) stage_a(i + 1);
        // ---- U = T R through 32-token halves (T is lower triangular), R as hi / lo ----
        // term by term over the blocks in the order (0,0) (1,0) (2,0) (3,0) (2,1) (3,1), so that
        // consecutive MFMAs update different tiles
        constexpr int kOrd[6] = {0, 1, 2, 4, 3, 5};  // block index p in that order
        cb::Split32 u0[CT], u1[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const cb::Split32 r0 = split_pair(Rr[c][0], Rr[c][1]), r1 = split_pair(Rr[c][2], Rr[c][3]);
            f32x4 U[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) U[rt] = zero4();
#pragma unroll
            for (int term = 0; term < 2; ++term)
#pragma unroll
                for (int q6 = 0; q6 < 6; ++q6) {
                    const int p = kOrd[q6];
                    const int rt = p < 2 ? p : 2 + (p - 2) / 2, k2 = p < 2 ? 0 : (p - 2) % 2;
                    const cb::Split32& rs = k2 == 0 ? r0 : r1;
                    mma(U[rt], ft[p], term == 0 ? rs.hi : rs.lo);
                }
            u0[c] = split_pair(U[0], U[1]);
            u1[c] = split_pair(U[2], U[3]);
        }
        // ---- S <- Gamma_C S + KG^T U, U as hi / lo: per 32-token half, the key-row fragments of
        // every tile, then each hi / lo term over all tiles (independent accumulators) ----
        const float* gc = reinterpret_cast<const float*>(rb + (R::GC - R::A_BYTES));
        const char* kh = rb + (R::KGT - R::A_BYTES);
#pragma unroll
        for (int st = 0; st < KT; ++st) {
            const f32x4 gv = *reinterpret_cast<const f32x4*>(gc + st * 16 + g4 * 4);
#pragma unroll
            for (int c = 0; c < CT; ++c) S[c][st] *= gv;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            Frag<bf16> fkh[KT];
#pragma unroll
            for (int st = 0; st < KT; ++st) fkh[st] = frag_perm(kh, st * 16 + l16, kk, g4, 128);
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const cb::Split32& us = kk == 0 ? u0[c] : u1[c];
#pragma unroll
                for (int st = 0; st < KT; ++st) mma(S[c][st], fkh[st], us.hi);
#pragma unroll
                for (int st = 0; st < KT; ++st) mma(S[c][st], fkh[st], us.lo);
            }
        }
        // ---- O = Y + P U, term by term over the blocks as for U ----
        if constexpr (MODE == kOut) {
            Frag<bf16> fph[6], fpl[6];
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const int rt = p < 2 ? p : 2 + (p - 2) / 2, k2 = p < 2 ? 0 : (p - 2) % 2;
                fph[p] = frag_tri(ph, rt * 16 + l16, k2, g4);
                fpl[p] = frag_tri(pl, rt * 16 + l16, k2, g4);
            }
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int term = 0; term < 3; ++term)
#pragma unroll
                    for (int q6 = 0; q6 < 6; ++q6) {
                        const int p = kOrd[q6];
                        const int rt = p < 2 ? p : 2 + (p - 2) / 2, k2 = p < 2 ? 0 : (p - 2) % 2;
                        const cb::Split32& us = k2 == 0 ? u0[c] : u1[c];
                        if (term == 0) mma(Y[c][rt], fph[p], us.hi);
                        else if (term == 1) mma(Y[c][rt], fph[p], us.lo);
                        else mma(Y[c][rt], fpl[p], us.hi);
                    }
        }
        // barrier F: this wave's loads (the next chunk's parts A and B, w and v, the previous
        // chunk's O stores) have drained; the barrier publishes every wave's and frees part B of
        // this chunk.  Then O, whose stores overlap the next chunk.
        __syncthreads();
        if constexpr (MODE == kOut) store_o(n, Y);
    }

    if constexpr (MODE == kTrans) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            float* dst = trans + ((int64_t)chain * D) * (2 * D) + slice * WGC + (wave * CT + c) * 16 + l16;
#pragma unroll
            for (int st = 0; st < KT; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)(st * 16 + g4 * 4 + r) * (2 * D)] = S[c][st][r];
        }
    } else {
        if (state_out && s0 + nb == nb_all) {
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int st = 0; st < KT; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        state_out[((int64_t)bh * D + st * 16 + g4 * 4 + r) * D + colc(c)] = S[c][st][r];
        }
    }
}

// Start states of the segments: S_0 the initial state (zero if none), copied, and
// S_g = A_{g-1} S_{g-1} + B_{g-1} (the transitions of the state kernel's kTrans mode, [D][2 D]
// per segment and head), written to starts[g] as [D][D].  One workgroup per (head, 16 state
// columns); the columns of a state are independent, so each workgroup walks the segments on
// its own, in fp32: wave w forms the 16-row tiles w, w + 4, .. of A_{g-1} S_{g-1} with fp32 MFMA
// (16 x 16 x 4), the rows of A_{g-1} as its A operands (four contraction steps per 16-byte load)
// and S_{g-1} transposed in LDS as the B operands; the next transition's rows load during the
// current step.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ trans, const float* s_init,
                                                      float* __restrict__ starts, int BH, int nseg) {
    constexpr int RT = D / 16;            // 16-row tiles of the state
    constexpr int TPW = (RT + 3) / 4;     // tiles per wave
    constexpr int KQ = D / 16;            // 16-wide contraction groups: k = 16 q + 4 g + e
    constexpr int SR = D + 4;             // floats per row of S^T in LDS (padded: distinct banks)
    __shared__ __attribute__((aligned(16))) float sT[2][16][SR];
    const int bh = blockIdx.x / (D / 16), ct = blockIdx.x % (D / 16);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    for (int x = tid; x < D * 16; x += 256) {
        const int r = x / 16, c = x % 16;
        const float v = s_init ? s_init[((int64_t)bh * D + r) * D + ct * 16 + c] : 0.f;
        starts[((int64_t)bh * D + r) * D + ct * 16 + c] = v;
        sT[0][c][r] = v;
    }
    // rows of A_{g-1} for this wave's tiles: lane (i, g) holds A[16 rt + i][16 q + 4 g .. + 3]
    auto load_a = [&](int g, f32x4 (&a)[TPW][KQ]) {
        const float* tr = trans + ((int64_t)(g - 1) * BH + bh) * D * (2 * D);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int rt = wave + 4 * t;
#pragma unroll
            for (int q = 0; q < KQ; ++q)
                a[t][q] = rt < RT ? *reinterpret_cast<const f32x4*>(tr + (int64_t)(16 * rt + l16) * (2 * D) + 16 * q + 4 * g4)
                                  : zero4();
        }
    };
    f32x4 a[TPW][KQ];
    if (nseg > 1) load_a(1, a);
    __syncthreads();
    for (int g = 1; g < nseg; ++g) {
        const int cur = (g - 1) & 1;
        f32x4 an[TPW][KQ];
        if (g + 1 < nseg) load_a(g + 1, an);
        const float* tr = trans + ((int64_t)(g - 1) * BH + bh) * D * (2 * D);
        f32x4 acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int rt = wave + 4 * t;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[t][r] = rt < RT ? tr[(int64_t)(16 * rt + 4 * g4 + r) * (2 * D) + D + ct * 16 + l16] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(&sT[cur][l16][16 * q + 4 * g4]);
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) mma_f32x4(acc[t], a[t][q][e], b[e]);
        }
        // S_g: lane (n, g) holds rows 16 rt + 4 g + r of column n
        float* dst = starts + ((int64_t)g * BH + bh) * D * D + ct * 16 + l16;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int rt = wave + 4 * t;
            if (rt < RT) {
                *reinterpret_cast<f32x4*>(&sT[cur ^ 1][l16][16 * rt + 4 * g4]) = acc[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * rt + 4 * g4 + r) * D] = acc[t][r];
            }
        }
        if (g + 1 < nseg) {
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int q = 0; q < KQ; ++q) a[t][q] = an[t][q];
        }
        __syncthreads();
    }
}

}  // namespace sp

// ------------------------------------------------------------------ host side ----
// Chunk-heads per batch: the records of one batch stay within the last-level cache.
constexpr int64_t kSplitBatchChunkHeads = 1024;

int64_t split_record_bytes(int64_t d) { return d == 128 ? sp::Rec<128>::BYTES : d == 64 ? sp::Rec<64>::BYTES : 0; }

int64_t split_batch_chunks(int64_t BH, int64_t nchunks) {
    int64_t c = kSplitBatchChunkHeads / (BH > 0 ? BH : 1);
    if (c < 1) c = 1;
    return c < nchunks ? c : nchunks;
}

// Segments of the few-chains form.  Each (sequence, head) is one chain of the state pass (one
// workgroup).  Cut into g segments of L chunks (at least 16), the form runs a transition pass
// (2 workgroups per chain and segment but the last) and then the forward pass (one per chain
// and segment), each L chunk steps long per round of workgroups over the compute units, plus a
// serial combine of g - 1 steps; in batches, each chain walks all its chunks.  Cost in chunk
// steps: batches ceil(chains / cus) nchunks; segments (transition rounds + forward rounds) L +
// 2 (g - 1).  The cheapest wins (two segments never do: they walk as many chunk steps as one).
// 1: the batched form.
int64_t split_segments(int64_t BH, int64_t nchunks, int64_t d, int64_t cus) {
    (void)d;  // a workgroup covers all dv columns at either head size
    const int64_t chains = BH;
    if (chains < 1 || cus < 1 || nchunks < 1) return 1;
    auto rounds = [&](int64_t wg) { return (wg + cus - 1) / cus; };
    int64_t best_g = 1, best = rounds(chains) * nchunks;
    for (int64_t g = 2; g <= nchunks / 16 && g <= 64; ++g) {
        const int64_t len = (nchunks + g - 1) / g;   // chunks per segment
        const int64_t gg = (nchunks + len - 1) / len;  // segments, none left empty
        const int64_t cost = (rounds(2 * (gg - 1) * chains) + rounds(gg * chains)) * len + 2 * (gg - 1);
        if (cost < best) {
            best = cost;
            best_g = gg;
        }
    }
    return best_g;
}

size_t split_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t cus) {
    const int64_t rb = split_record_bytes(d);
    if (rb == 0 || B < 1 || T < 1 || H < 1) return 0;
    const int64_t nc = (T + 63) / 64, BH = B * H;
    const int64_t g = split_segments(BH, nc, d, cus);
    if (g > 1)  // every chunk's record, the transitions of segments 0 .. g - 2, every start state
        return (size_t)(BH * nc * rb + (g - 1) * BH * d * (2 * d) * 4 + g * BH * d * d * 4);
    const int64_t bc = split_batch_chunks(BH, nc);
    // records of one batch, then the state carried between batches
    return (size_t)(BH * bc * rb + BH * d * d * 4);
}

template <typename OutT, int D, typename Gt>
hipError_t launch_split_d(const ChunkArgs& a, char* ws) {
    const int64_t BH = a.B * a.H;
    const int nc = (int)((a.T + 63) / 64);
    const int nslices = D / sp::StateCfg<D>::WGC;  // 1: a workgroup covers all value columns
    hipStream_t st = (hipStream_t)a.stream;
    const int g = (int)split_segments(BH, nc, D, a.cus);
    if (g > 1) {
        const int len = (nc + g - 1) / g;
        char* trans = ws + BH * nc * sp::Rec<D>::BYTES;
        float* tr = reinterpret_cast<float*>(trans);
        float* starts = tr + (int64_t)(g - 1) * BH * D * 2 * D;
        // every chunk's record, in one launch: runs of at least 8 chunks in about four rounds of
        // workgroups, so that the hardware's dispatch evens out chunks of unequal cost (a
        // strong-decay chunk takes about twice a mild one, and whole heads can be strong)
        const int64_t per0 = (BH * nc + 4 * (int64_t)a.cus - 1) / (4 * (int64_t)a.cus);
        const int64_t per = per0 < 8 ? 8 : per0;
        const int run = (int)(per > nc ? nc : per);
        const int runs = (nc + run - 1) / run;
        hipLaunchKernelGGL((sp::local_kernel<D, Gt>), dim3((unsigned)(BH * runs)), dim3(sp::NT_LOCAL), 0, st,
                           (const bf16*)a.q, (const bf16*)a.k, (const typename Gt::Decay*)a.decay(),
                           (const bf16*)a.b, ws, (int)a.T, (int)a.H, 0, nc, run);
        // the transitions of segments 0 .. g - 2
        const int64_t tchains = (int64_t)(g - 1) * BH;
        hipLaunchKernelGGL((sp::state_kernel<OutT, D, Gt, sp::kTrans>), dim3((unsigned)(tchains * 2 * nslices)),
                           dim3(sp::NT_STATE), 0, st, (const char*)ws, (const bf16*)a.v, (const bf16*)a.w,
                           (const float*)nullptr, (float*)nullptr, (OutT*)nullptr, (int)a.T, (int)a.H, nslices,
                           tchains % 8 == 0 ? 1 : 0, 0, nc, (int)BH, len, (const float*)nullptr, tr);
        hipLaunchKernelGGL((sp::combine_kernel<D>), dim3((unsigned)(BH * (D / 16))), dim3(256), 0, st,
                           (const float*)tr, a.initial_state, starts, (int)BH, g);
        const int64_t chains = (int64_t)g * BH;
        hipLaunchKernelGGL((sp::state_kernel<OutT, D, Gt, sp::kOut>), dim3((unsigned)(chains * nslices)),
                           dim3(sp::NT_STATE), 0, st, (const char*)ws, (const bf16*)a.v, (const bf16*)a.w,
                           a.initial_state, a.final_state, (OutT*)a.o, (int)a.T, (int)a.H, nslices,
                           chains % 8 == 0 ? 1 : 0, 0, nc, (int)BH, len, (const float*)starts, (float*)nullptr);
        return hipGetLastError();
    }
    const int bc = (int)split_batch_chunks(BH, nc);
    const int xcd_map = BH % 8 == 0 ? 1 : 0;
    float* carry = a.final_state ? a.final_state : reinterpret_cast<float*>(ws + BH * bc * sp::Rec<D>::BYTES);
    for (int c0 = 0; c0 < nc; c0 += bc) {
        const int c1 = c0 + bc < nc ? c0 + bc : nc;
        // runs of consecutive chunks per local workgroup: one round of workgroups over the CUs
        const int64_t per = (BH * (c1 - c0) + a.cus - 1) / a.cus;
        const int run = (int)(per < 1 ? 1 : per > c1 - c0 ? c1 - c0 : per);
        const int runs = (c1 - c0 + run - 1) / run;
        hipLaunchKernelGGL((sp::local_kernel<D, Gt>), dim3((unsigned)(BH * runs)), dim3(sp::NT_LOCAL), 0, st,
                           (const bf16*)a.q, (const bf16*)a.k, (const typename Gt::Decay*)a.decay(),
                           (const bf16*)a.b, ws, (int)a.T, (int)a.H, c0, c1, run);
        const float* sin = c0 == 0 ? a.initial_state : carry;
        float* sout = c1 == nc ? a.final_state : carry;
        hipLaunchKernelGGL((sp::state_kernel<OutT, D, Gt, sp::kOut>), dim3((unsigned)(BH * nslices)),
                           dim3(sp::NT_STATE), 0, st, (const char*)ws, (const bf16*)a.v, (const bf16*)a.w, sin,
                           sout, (OutT*)a.o, (int)a.T, (int)a.H, nslices, xcd_map, c0, c1, (int)BH, c1 - c0,
                           (const float*)nullptr, (float*)nullptr);
    }
    return hipGetLastError();
}

template <typename OutT, int D>
hipError_t launch_split_g(const ChunkArgs& a, char* ws) {
    return a.gate_logits ? launch_split_d<OutT, D, GatesLogits>(a, ws) : launch_split_d<OutT, D, GatesActivated>(a, ws);
}

hipError_t launch_chunk_split(const ChunkArgs& a, void* workspace) {
    char* ws = static_cast<char*>(workspace);
    if (!a.dtype_bf16 || a.dk != a.dv || a.cu_seqlens) return hipErrorInvalidValue;
    if (a.dk == 128) return a.out_f32 ? launch_split_g<float, 128>(a, ws) : launch_split_g<bf16, 128>(a, ws);
    if (a.dk == 64) return a.out_f32 ? launch_split_g<float, 64>(a, ws) : launch_split_g<bf16, 64>(a, ws);
    return hipErrorInvalidValue;
}

}  // namespace gdn2
