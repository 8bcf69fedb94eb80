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
//     with hi + lo bf16 MFMA products, and the diagonal block of P beside it; waves 4-6 form
//     the off-diagonal blocks.
//   * the off-diagonal blocks of T = (I + A)^{-1} through halves of 32 tokens:
//     T = [[T_A, 0], [T_C, T_B]], T_10 = -T_11 A_10 T_00, T_32 likewise, T_C = -T_B A_BA T_A.
//   * the state: wave 4 + j holds the 16 value columns j of the slice, all key rows, in fp32
//     MFMA accumulators for the whole sequence.  While waves 0-3 form T_C, it forms
//     Z = ((b.k).Gamma) S and Y = (q.Gamma) S, which need no T; then, in its own registers,
//     U = T (w.v - Z) (= U0 - W S of the formulas above, with the product regrouped),
//     O = Y + P U and S_next.  Waves 0-3 meanwhile start the next chunk.
// Operands that are not bf16 numbers themselves (w.v - Z, U, P) enter the MFMAs as hi + lo
// bf16 pairs, and so does k / Gamma in P on the single-pivot path (its rounding is the
// largest single source of the output's error there); every product accumulates in fp32.

#include "gdn2_bf16_ops.h"
#include "gdn2_launch.h"

namespace gdn2 {
namespace cb {

constexpr int NT = 512;

template <int DK, int DVS>
struct Cfg {
    static constexpr int CPL = DK / 32;   // key channels per lane in the element phase
    static constexpr int KT = DK / 16;    // 16-channel tiles
    static constexpr int NCT = DVS / 16;  // 16-column value tiles of the slice: one state wave each
    static constexpr int LDK = DK + 8;    // bf16 row stride of [token][channel] tiles
    static constexpr int LC = C + 8;      // bf16 row stride of [*][token] tiles
    static constexpr int VC = C * DVS / NT >= 4 ? 4 : C * DVS / NT;  // value columns per lane
    static constexpr int TPV = C * DVS / (NT * VC);                  // value tokens per lane
    // LDS regions (byte offsets); lifetimes within a chunk in the comments
    static constexpr int QG = 0;                              // [64][LDK] q.Gamma: element -> Y
    static constexpr int KGT = QG + C * LDK * 2;              // [DK][LC] (k.Gamma')^T: element -> state update
    static constexpr int BG = KGT + DK * LC * 2;              // [64][LDK] (b.k).Gamma: element -> A (mild), Z
    static constexpr int WVT = BG + C * LDK * 2;              // [DVS][64] fp32 (w.v)^T (16-byte units
                                                              // swizzled by wv_swz): element -> state pass
    static constexpr int PM = WVT + DVS * C * 4;              // 2 x [64][LC] P hi, lo: A,P -> O
    static constexpr int AM = PM + 2 * C * LC * 2;            // [64][LC] -A_IJ (J < I), (I + A_II)^{-1}
    static constexpr int RX = AM + C * LC * 2;                // work area, 192 rows of [LDK]:
                                                              //   mild: K/Gamma hi rows 64-127, lo 0-63
                                                              //   strong: group and level tiles
                                                              //   T = (I + A)^{-1} rows 128-
    static constexpr int TR = RX + 2 * C * LDK * 2;           // [64][LC] T, row-major: -> state pass
    static constexpr int GC = RX + 192 * LDK * 2;             // [DK] fp32 whole-chunk decays
    static constexpr int BLK = GC + DK * 4;                   // [4][DK] fp32 16-token block decays
    static constexpr int FLG = BLK + 4 * DK * 4;              // [8] int: per-wave strong-decay votes
    static constexpr int TTR = FLG + 8 * 4;                   // [64][LC] T^T (blocks of T_A and T_22)
    static constexpr int BYTES = TTR + C * LC * 2;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(BYTES >= 4 * (kMaxSort + 1), "no room for the sequence order");
    static_assert(TR + C * LC * 2 <= GC, "T does not fit the work area");
    static_assert(DK % 64 == 0 && DVS % 16 == 0 && DVS <= 64 && TPV >= 1, "shape");
};

// An operand fragment in the permuted slot map of a pair of accumulator tiles: slot (g, e) of
// the 32-wide contraction block holds element 4 g + e for e < 4 and 16 + 4 g + e - 4 above, so
// that a pair of 16 x 16 accumulators (lane holds rows 4 g .. 4 g + 3 of each) is directly an
// operand.  p points at element 4 g of the block's row; two 8-byte halves.
__device__ __forceinline__ Frag<bf16> load_halves(const bf16* p) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
    Frag<bf16> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.v[e] = a[e];
        f.v[e + 4] = b[e];
    }
    return f;
}

// Unpadded [column][token] fp32 rows of 64 tokens (256 bytes): the 16-byte unit u (4 tokens) of
// row r sits at unit u ^ wv_swz(r).  The swizzle is one-to-one on 16 consecutive rows (the state
// pass's reads) and on 16 rows 4 apart (the element phase's stores), so both fall on distinct
// banks.
__device__ __forceinline__ int wv_swz(int r) { return (r ^ (r >> 2)) & 15; }

// Inputs of one chunk as one thread loads them: CPL key channels of 4 tokens, and VC value
// columns of TPV tokens.
template <int CPL, int TPV, int VC, typename Decay>
struct In {
    Raw<Decay, CPL> g[4];
    Raw<bf16, CPL> q[4], k[4], b[4];
    Raw<bf16, VC> w[TPV], v[TPV];
};

template <typename OutT, int DK, int DV, int DVS, typename Gt>
__global__ __launch_bounds__(NT) void chunk_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const typename Gt::Decay* __restrict__ decay, const bf16* __restrict__ bgate, const bf16* __restrict__ wgate,
    const float* initial_state, OutT* __restrict__ o, float* final_state, int B, int Tparam, int H,
    int nslices, int xcd_map, const int64_t* __restrict__ cu_seqlens) {
    using G = Cfg<DK, DVS>;
    constexpr int CPL = G::CPL, KT = G::KT, NCT = G::NCT;
    constexpr int LDK = G::LDK, LC = G::LC, VC = G::VC, TPV = G::TPV;
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

    // ---- the state slice in accumulators: wave 4 + j (j < NCT) holds value columns 16 j ..
    // 16 j + 15 of the slice for every key row, as KT tiles; lane (n, g) of tile st holds
    // S[16 st + 4 g + r][16 j + n] ----
    const int sct = wave - 4;
    const bool owner = sct >= 0 && sct < NCT;  // uniform across the wave
    const int sc = owner ? sct : 0;
    f32x4 S[KT];
#pragma unroll
    for (int i = 0; i < KT; ++i) S[i] = zero4();
    if (initial_state && owner) {
#pragma unroll
        for (int st = 0; st < KT; ++st) {
            const float* src = initial_state + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + sc * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[st][r] = src[(int64_t)r * DV];
        }
    }

    const int nchunks = (Tlen + C - 1) / C;
    const int64_t tok_stride_k = (int64_t)H * DK;
    const int64_t tok_stride_v = (int64_t)H * DV;
    const int64_t seq_base_k = (tok0 * H + h) * DK;
    const int64_t seq_base_v = (tok0 * H + h) * DV;

    // The next chunk's inputs are loaded in two batches (decays; queries, keys, gates and values:
    // fewer registers held through the T_C step), each issued well before it is needed and
    // without a branch.  Each array is read through a buffer resource over the chunk's tokens of
    // this head: a token past the end of the sequence reads zeros (k = 0, and for activated gates
    // log alpha = 0, no decay).
    // Offsets: (token * H * D + channel) * element size from the chunk's first token; the host
    // keeps H * D below 2^22, so offsets and the buffer range stay below 2^30 bytes.
    const int rsk = H * DK, rsv = H * DV;  // elements between consecutive tokens
    using Decay = typename Gt::Decay;
    using InC = In<CPL, TPV, VC, Decay>;
    auto load_first = [&](int n, InC& in) {
        const int t0 = n * C, ntok = min(C, Tlen - t0);
        const int64_t cb = seq_base_k + (int64_t)t0 * tok_stride_k;
        const auto rg = buffer_over(decay + cb, ntok * rsk * (int)sizeof(Decay));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t e = __umul24(I * 16 + ts * 4 + m, rsk) + c0;
            in.g[m] = bload_raw<Decay, CPL>(rg, e * (uint32_t)sizeof(Decay));
        }
    };
    auto load_second = [&](int n, InC& in) {
        const int t0 = n * C, ntok = min(C, Tlen - t0);
        const int64_t cb = seq_base_k + (int64_t)t0 * tok_stride_k;
        const auto rq = buffer_over(q + cb, ntok * rsk * 2);
        const auto rk = buffer_over(k + cb, ntok * rsk * 2);
        const auto rb = buffer_over(bgate + cb, ntok * rsk * 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t e = __umul24(I * 16 + ts * 4 + m, rsk) + c0;
            in.q[m] = bload_raw<bf16, CPL>(rq, e * 2);
            in.k[m] = bload_raw<bf16, CPL>(rk, e * 2);
            in.b[m] = bload_raw<bf16, CPL>(rb, e * 2);
        }
        const int64_t cv = seq_base_v + (int64_t)t0 * tok_stride_v + col0;
        const auto rw = buffer_over(wgate + cv, ntok * rsv * 2);
        const auto rv = buffer_over(v + cv, ntok * rsv * 2);
#pragma unroll
        for (int i = 0; i < TPV; ++i) {
            const uint32_t e = __umul24(vtok + i, rsv) + vcol;
            in.w[i] = bload_raw<bf16, VC>(rw, e * 2);
            in.v[i] = bload_raw<bf16, VC>(rv, e * 2);
        }
    };

    InC in;
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
        // Tokens past the end of the sequence (read as zeros) act as the identity: k = 0 zeroes
        // their A, P-column, BG and KG entries, and their decay is 1 (a zero log alpha is;
        // a zero logit is not, and is replaced).
        bool tok_ok[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) tok_ok[m] = Gt::zero_is_identity || t0 + I * 16 + ts * 4 + m < Tlen;
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
                    al[m] = tok_ok[m] ? Gt::alpha(in.g[m].f(c)) : 1.f;
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
        lds_barrier();

        // =============== element phase, pass 2: scaled operands ===============
        // the gate and value registers are first read here (kept from being read earlier: the
        // wait for their loads then falls after the first pass)
#pragma unroll
        for (int i = 0; i < TPV; ++i)
#pragma unroll
            for (int j = 0; j < Raw<bf16, VC>::W; ++j) asm volatile("" : "+v"(in.w[i].u[j]), "+v"(in.v[i].u[j]));
        // gate times value, transposed ([column][token]), in fp32 (exact: the product of two bf16
        // numbers has at most 16 significant bits).  Here rather than in pass 1: w and v are the
        // later of the two batches of loads, and pass 1 then waits for the first batch only.
#pragma unroll
        for (int j = 0; j < VC; ++j) {
            const int row = vcol + j;
            const int wvb = opq(G::WVT + row * C * 4 + ((((vtok >> 2) ^ wv_swz(row)) << 2) | (vtok & 3)) * 4);
            typedef float V __attribute__((ext_vector_type(TPV)));
            V x;
#pragma unroll
            for (int i = 0; i < TPV; ++i) x[i] = Gt::gate(in.w[i].f(j)) * in.v[i].f(j);
            *reinterpret_cast<V*>(__builtin_assume_aligned(smem + wvb, 4 * TPV)) = x;
        }
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
            float kgt[CPL][4];
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
                        const float kv = in.k[m].f(c);
                        const float gam = bex[c] * lp[c][m];
                        xq[c] = in.q[m].f(c) * gam;
                        xb[c] = Gt::gate(in.b[m].f(c)) * kv * gam;
                        kgt[c][m] = kv * (ls[c][m] * esa[c]);
                        xki[c] = kgt[c][m] * invgc[c];
                    }
                    store_bf16<CPL>(B16(eb + m * LDK * 2), xq);
                    store_bf16<CPL>(B16(eb + G::BG + m * LDK * 2), xb);
                    // KI as a hi/lo pair: hi in work rows 64-127, lo in rows 0-63 (free on this path)
                    store_bf16_split<CPL>(B16(ebx + (C + m) * LDK * 2), B16(ebx + m * LDK * 2), xki);
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
                    float xq[CPL], xb[CPL], ya[CPL], yp[CPL], za[CPL], zp[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float qv = in.q[m].f(c);
                        const float kv = in.k[m].f(c);
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
                    store_bf16<CPL>(B16(eb + m * LDK * 2), xq);
                    store_bf16<CPL>(B16(eb + G::BG + m * LDK * 2), xb);
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
            for (int c = 0; c < CPL; ++c) store_bf16<4>(B16(tb + c * LC * 2), kgt[c]);
        }
        lds_barrier();


        // =============== A, P and the diagonal blocks of T = (I + A)^{-1} ===============
        if (!strong) {
            load_first(nnext, in);
            // single pivot at the chunk start: A = BG KI^T, P = QG KI^T on the lower blocks
            // (wave 7 has no part here)
            if (wave < 4) {
                // diagonal block I = wave: A_II in both orientations, then its inverse, and P_II
                f32x4 nt = zero4(), nn = zero4();
                const int rk = opq(((wave * 16 + l16) * LDK + g4 * 8) * 2);
                Frag<bf16> fk[DK / 32], fa[DK / 32], fq[DK / 32], fl[DK / 32];
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    fk[kk] = load_contig(B16(rk + G::RX + C * LDK * 2 + kk * 64));
                    fa[kk] = load_contig(B16(rk + G::BG + kk * 64));
                    fq[kk] = load_contig(B16(rk + kk * 64));
                    fl[kk] = load_contig(B16(rk + G::RX + kk * 64));  // KI lo
                }
                sched_fence();
                f32x4 pd = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    mma(nt, fk[kk], fa[kk]);  // lane holds A[l16][4 g4 + r]
                    mma(nn, fa[kk], fk[kk]);  // lane holds A[4 g4 + r][l16]
                }
                // the diagonal block of P beside it (independent of the inverse's chain)
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    mma(pd, fk[kk], fq[kk]);  // P[l16][4 g4 + r]
                    mma(pd, fl[kk], fq[kk]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * g4 + r;
                    nt[r] = j < l16 ? nt[r] : 0.f;
                    nn[r] = j > l16 ? nn[r] : 0.f;
                }
                store_tdiag<G>(smem, wave, l16, g4, unit_lower_inverse(nt, nn, l16, g4));
                float pp[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) pp[r] = 4 * g4 + r <= l16 ? pd[r] : 0.f;
                const int idx = (wave * 16 + l16) * LC + wave * 16 + g4 * 4;
                store_bf16_split<4>(sPh + idx, sPl + idx, pp);
            } else if (wave < 7) {
                // off-diagonal pairs, two per wave sharing a block row or column:
                // wave 4: (1,0) (2,0); wave 5: (2,1) (3,1); wave 6: (3,0) (3,2)
                const int rl = opq((l16 * LDK + g4 * 8) * 2);
#pragma unroll
                for (int pi = 0; pi < 2; ++pi) {
                    const int Ib = wave == 4 ? 1 + pi : wave == 5 ? 2 + pi : 3;
                    const int Jb = wave == 4 ? 0 : wave == 5 ? 1 : 2 * pi;
                    f32x4 accA = zero4(), accP = zero4();
                    Frag<bf16> fk[DK / 32], fl[DK / 32], fa[DK / 32], fq[DK / 32];
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        fk[kk] = load_contig(B16(rl + G::RX + (C + Jb * 16) * LDK * 2 + kk * 64));
                        fa[kk] = load_contig(B16(rl + G::BG + Ib * 16 * LDK * 2 + kk * 64));
                        fq[kk] = load_contig(B16(rl + Ib * 16 * LDK * 2 + kk * 64));
                        fl[kk] = load_contig(B16(rl + G::RX + Jb * 16 * LDK * 2 + kk * 64));  // KI lo
                    }
                    sched_fence();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk) {
                        mma(accA, fk[kk], fa[kk]);
                        mma(accP, fk[kk], fq[kk]);
                        mma(accP, fl[kk], fq[kk]);
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
            // the next chunk's first loads go out before the call (the strong path reads its
            // inputs from global memory): issued after it, they would leave the compiler unable to
            // count the loads in flight at the top of the loop, and it would wait for all of them
            load_first(nnext, in);
            strong_ap<G, DK, Gt>(smem, q, k, bgate, decay, seq_base_k + (int64_t)t0 * tok_stride_k, tok_stride_k,
                             Tlen - t0, [&](int row, int col, const float (&p)[4]) {
                                 const int idx = row * LC + col;
                                 store_bf16_split<4>(sPh + idx, sPl + idx, p);
                             }, [](int, const f32x4&) {});
        }
        lds_barrier();

        // =============== off-diagonal blocks of T, through halves of 32 tokens ===============
        // (waves 0-3; the state waves meanwhile form Z and Y)
        f32x4 Z[4], Y[4];
        // T = [[T_A, 0], [T_C, T_B]] with T_A = [[T_00, 0], [T_10, T_11]], T_B likewise, and
        // T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22, T_C = -T_B A_BA T_A.  The local store
        // holds -A, so every product below adds.  B operands that are columns of T come from T^T.
        if (wave < 4) {
            // the next chunk's keys, gates and values, issued ahead of the state waves' share: the
            // CU's load issue is a queue, and these waves have time to spare in this step
            load_second(nnext, in);
            // block (R, J) of T_C, one per wave: Z_xJ = (-A_x0) T_0J + (-A_x1) T_1J, then
            // T_2J = T_22 Z_2J and T_3J = T_32 Z_2J + T_33 Z_3J, formed transposed so that
            // lane (i, g) holds a row: T_RJ[i][4 g + r].  T_10 (needed for J = 0) and T_32 (for
            // R = 3) come from the diagonal blocks alone; the waves that need them form them here
            // (waves 0 and 3 also store them for the state pass), so no level of their own
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
        } else {
            if (owner) {
                // Z = BG S and Y = QG S for this wave's 16 value columns, which need no T.  Pairs of
                // state tiles are the B operands as they stand (slot map of load_halves); the rows of
                // BG and QG are read in the same map.  Z: lane (n, g) holds Z[16 rt + 4 g + r][n];
                // Y: lane (i, g) holds Y[16 rt + i][4 g + r], the orientation of the o stores.
                Frag<bf16> sf[KT / 2];
#pragma unroll
                for (int m = 0; m < KT / 2; ++m) sf[m] = frag_from_acc<bf16>(S[2 * m], S[2 * m + 1]);
                const int rb = opq((l16 * LDK + g4 * 4) * 2);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    Frag<bf16> fb[KT / 2], fq[KT / 2];
#pragma unroll
                    for (int m = 0; m < KT / 2; ++m) {
                        fb[m] = load_halves(B16(G::BG + rb + (rt * 16 * LDK + m * 32) * 2));
                        fq[m] = load_halves(B16(G::QG + rb + (rt * 16 * LDK + m * 32) * 2));
                    }
                    sched_fence();
                    Z[rt] = zero4();
                    Y[rt] = zero4();
#pragma unroll
                    for (int m = 0; m < KT / 2; ++m) {
                        mma(Z[rt], fb[m], sf[m]);
                        mma(Y[rt], sf[m], fq[m]);
                    }
                }
            }
            load_second(nnext, in);
        }

        lds_barrier();

        // =============== state pass: this wave's 16 value columns ===============
        // R = w.v - Z, U = T R, O = Y + P U, S <- Diag(Gamma_C) S + KG^T U, all in this wave's
        // registers: an accumulator pair (16 tokens apart) is the next product's B operand in the
        // slot map of load_halves, so R and U never go through LDS.  No barrier follows: waves 0-3
        // go on to the next chunk's first element pass, which writes only the votes and the block
        // decays; the barrier after it keeps the next operand tiles behind these reads.
        if (owner) {
            const int row = sc * 16 + l16;  // this lane's value column: a row of (w.v)^T
            const int wb = opq(G::WVT + row * C * 4);
            const int ws = wv_swz(row);
            const int rl = opq((l16 * LC + g4 * 4) * 2);
            f32x4 wv[4];
            Frag<bf16> tf[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                // tokens 16 rt + 4 g .. + 3: 16-byte unit 4 rt + g
                wv[rt] = *reinterpret_cast<const f32x4*>(smem + wb + (((4 * rt + g4) ^ ws) << 4));
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (m > rt / 2) continue;
                    tf[rt][m] = load_halves(B16(G::TR + rl + (rt * 16 * LC + m * 32) * 2));
                }
            }
            sched_fence();
            f32x4 R[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) R[rt][r] = wv[rt][r] - Z[rt][r];
            const Split32 rs[2] = {split32(R[0], R[1]), split32(R[2], R[3])};
            // U = T R: lane (n, g) holds U[16 rt + 4 g + r][n]
            f32x4 U[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                U[rt] = zero4();
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (m > rt / 2) continue;
                    mma(U[rt], tf[rt][m], rs[m].hi);
                    mma(U[rt], tf[rt][m], rs[m].lo);
                }
            }
            const Split32 us[2] = {split32(U[0], U[1]), split32(U[2], U[3])};
            // O = Y + P U, in Y's orientation (lane (i, g): O[16 rt + i][4 g + r])
            Frag<bf16> ph[4][2], pl[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (m > rt / 2) continue;
                    ph[rt][m] = load_halves(B16(G::PM + rl + (rt * 16 * LC + m * 32) * 2));
                    pl[rt][m] = load_halves(B16(G::PM + rl + (C * LC + rt * 16 * LC + m * 32) * 2));
                }
            sched_fence();
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (m > rt / 2) continue;
                    mma(Y[rt], us[m].hi, ph[rt][m]);
                    mma(Y[rt], us[m].lo, ph[rt][m]);
                    mma(Y[rt], us[m].hi, pl[rt][m]);
                }
            // S <- Diag(Gamma_C) S + KG^T U, in two halves of the row tiles; KG^T's rows are
            // swizzled by 16-byte units: unit u of row 16 st + i sits at u ^ st
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                Frag<bf16> kf[KT / 2][2];
#pragma unroll
                for (int j = 0; j < KT / 2; ++j) {
                    const int st = h2 * (KT / 2) + j;
                    const int kb = opq(G::KGT + (st * 16 + l16) * LC * 2 + ((g4 & 1) << 3));
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const bf16x4 a = *reinterpret_cast<const bf16x4*>(
                            smem + kb + ((((4 * m + (g4 >> 1)) ^ st) & 7) << 4));
                        const bf16x4 b = *reinterpret_cast<const bf16x4*>(
                            smem + kb + ((((4 * m + 2 + (g4 >> 1)) ^ st) & 7) << 4));
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            kf[j][m].v[e] = a[e];
                            kf[j][m].v[e + 4] = b[e];
                        }
                    }
                }
                sched_fence();
#pragma unroll
                for (int j = 0; j < KT / 2; ++j) {
                    const int st = h2 * (KT / 2) + j;
                    S[st] *= *reinterpret_cast<const f32x4*>(sGC + st * 16 + g4 * 4);
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        mma(S[st], kf[j][m], us[m].hi);
                        mma(S[st], kf[j][m], us[m].lo);
                    }
                }
            }
        }
        // o through a buffer resource over this chunk's tokens of the head: a last partial chunk's
        // rows past the end of the sequence fall outside its range and are dropped, and so is
        // everything a wave without state columns issues (range 0).  The stores therefore sit on
        // no branch (behind one, the compiler would assume a path where they are not in flight
        // and wait for every load at the top of the next chunk).
        {
            const int ntok = min(C, Tlen - t0);
            const auto ro = __builtin_amdgcn_make_buffer_rsrc(o + seq_base_v + (int64_t)t0 * tok_stride_v, 0,
                                                              owner ? ntok * rsv * (int)sizeof(OutT) : 0, 0x00020000);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const uint32_t e = (__umul24(rt * 16 + l16, rsv) + col0 + sc * 16 + g4 * 4) * sizeof(OutT);
                if constexpr (sizeof(OutT) == 4) {
                    typedef uint32_t U4 __attribute__((ext_vector_type(4)));
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(U4, Y[rt]), ro, (int)e, 0, 0);
                } else {
                    typedef uint32_t U2 __attribute__((ext_vector_type(2)));
                    bf16x4 y;
#pragma unroll
                    for (int r = 0; r < 4; ++r) y[r] = (bf16)Y[rt][r];
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(U2, y), ro, (int)e, 0, 0);
                }
            }
        }
    }

    if (owner && final_state) {
#pragma unroll
        for (int st = 0; st < KT; ++st) {
            float* dst = final_state + ((int64_t)bh * DK + st * 16 + g4 * 4) * DV + col0 + sc * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)r * DV] = S[st][r];
        }
    }
}

template <typename OutT, int D, int DVS, typename Gt>
hipError_t launch(const ChunkArgs& a) {
    const int nslices = D / DVS;
    const int64_t groups = (int64_t)a.B * a.H * nslices;
    const int xcd_map = ((int64_t)a.B * a.H) % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((chunk_bf16_kernel<OutT, D, D, DVS, Gt>), dim3((unsigned)groups), dim3(NT), 0,
                       (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       (const typename Gt::Decay*)a.decay(), (const bf16*)a.b, (const bf16*)a.w,
                       a.initial_state, (OutT*)a.o, a.final_state, (int)a.B, (int)a.T, (int)a.H, nslices,
                       xcd_map, a.cu_seqlens);
    return hipGetLastError();
}

template <typename OutT, int D, typename Gt>
hipError_t launch_dvs(const ChunkArgs& a, int dvs) {
    switch (dvs) {
        case 16: return launch<OutT, D, 16, Gt>(a);
        case 32: return launch<OutT, D, 32, Gt>(a);
        case 64: return launch<OutT, D, 64, Gt>(a);
    }
    return hipErrorInvalidValue;
}

template <typename OutT, int D>
hipError_t launch_gates(const ChunkArgs& a, int dvs) {
    return a.gate_logits ? launch_dvs<OutT, D, GatesLogits>(a, dvs) : launch_dvs<OutT, D, GatesActivated>(a, dvs);
}

}  // namespace cb

hipError_t launch_chunk_bf16(const ChunkArgs& a, int dvs) {
    if (a.dk != a.dv || !a.dtype_bf16) return hipErrorInvalidValue;
    if (a.dk == 128) return a.out_f32 ? cb::launch_gates<float, 128>(a, dvs) : cb::launch_gates<bf16, 128>(a, dvs);
    if (a.dk == 64) return a.out_f32 ? cb::launch_gates<float, 64>(a, dvs) : cb::launch_gates<bf16, 64>(a, dvs);
    return hipErrorInvalidValue;
}

}  // namespace gdn2
