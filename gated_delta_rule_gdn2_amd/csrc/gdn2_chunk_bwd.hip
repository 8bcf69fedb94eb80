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
// Three launches:
//   1. bwd_fwd_kernel, one workgroup per (sequence, head, slice of value columns): the forward
//      re-run in fp32 from the inputs (A, P, T = (I + A)^{-1} formed again), storing the state
//      entering every chunk, U, and T and P of every chunk;
//   2. bwd_state_kernel, one workgroup per (sequence, head, slice of value columns): the
//      chunks in reverse order with dS in MFMA accumulators; stores dS' of every chunk, dR,
//      and dS of the first chunk (the gradient of the initial state);
//   3. bwd_chunk_kernel, one workgroup per (sequence, head, chunk): every gradient of the
//      chunk's inputs, independently of the other chunks.
// Products run on fp32 MFMA (v_mfma_f32_16x16x4_f32) with fp32 accumulation.
//
// Decays in kernels 1 and 3: a chunk whose whole-chunk decay stays >= e^-40 on every channel
// pivots all factors at the chunk start (k / Gamma is then finite, and every masked product is
// one MFMA pass); any other chunk forms its masked sums element by element from
// e^{G_i - G_j}, which never exceeds 1.
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

// acc += sum_{k in [k0, k1)} A(m, k) B(k, n) over one 16 x 16 tile, k0 and k1 multiples of 16:
// lane (n = l16, g4) supplies A(l16, k + g4) and B(k + g4, l16) at each step of 4.
template <class FA, class FB>
__device__ __forceinline__ void mm(f32x4& acc, FA A, FB B, int k0, int k1, int l16, int g4) {
    for (int k = k0; k < k1; k += 16) {
#pragma unroll
        for (int s = 0; s < 16; s += 4) acc = mfma4(acc, A(l16, k + s + g4), B(k + s + g4, l16));
    }
}

// NTILE independent 16 x 16 products over the same contraction length K (compile time), fully
// unrolled with the steps of all tiles interleaved, so that the MFMA chains of different tiles
// hide each other's latency: acc[t] += sum_k A(t, m, k) B(t, k, n).  A B operand that does not
// depend on t is loaded once per step.
template <int NTILE, int K, class FA, class FB>
__device__ __forceinline__ void mm_n(f32x4 (&acc)[NTILE], FA A, FB B, int l16, int g4) {
    // unrolled 16 deep: deeper unrolling lets the compiler hoist more operand loads than the
    // register file holds
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
        for (int k = k0; k < k0 + 16; k += 4) {
            float a[NTILE], b[NTILE];
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
                a[t] = A(t, l16, k + g4);
                b[t] = B(t, k + g4, l16);
            }
#pragma unroll
            for (int t = 0; t < NTILE; ++t) acc[t] = mfma4(acc[t], a[t], b[t]);
        }
    }
}

// acc += the product over [0, K) as NS independent chains over consecutive parts of K, summed
// at the end (one output tile, its MFMA latency hidden by its own parts)
template <int NS, int K, class FA, class FB>
__device__ __forceinline__ void mm_split(f32x4& acc, FA A, FB B, int l16, int g4) {
    static_assert(K % (4 * NS) == 0, "split");
    f32x4 part[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) part[t] = zero4();
    mm_n<NS, K / NS>(part, [&](int t, int m, int kk) { return A(m, t * (K / NS) + kk); },
                     [&](int t, int kk, int nn) { return B(t * (K / NS) + kk, nn); }, l16, g4);
#pragma unroll
    for (int t = 0; t < NS; ++t) acc += part[t];
}

// acc += the product over the 16-wide blocks kb0 <= kb < 4 of a 64-long contraction (kb0
// runtime), each block its own chain
template <class FA, class FB>
__device__ __forceinline__ void mm_tail64(f32x4& acc, FA A, FB B, int kb0, int l16, int g4) {
    f32x4 part[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) part[t] = zero4();
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t >= kb0) part[t] = mfma4(part[t], A(l16, t * 16 + k + g4), B(t * 16 + k + g4, l16));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) acc += part[t];
}

// This thread's L tokens of key channel c in the element phase, every load issued at once: a
// token past the end reads the last token, and the caller zeroes it.
template <typename In, int L>
struct KeyIn {
    float g[L];
    In q[L], k[L], b[L];
};
template <typename In, int L>
__device__ __forceinline__ void load_key(KeyIn<In, L>& in, const In* __restrict__ q, const In* __restrict__ k,
                                         const In* __restrict__ b, const float* __restrict__ g, int64_t base,
                                         int64_t rk, int t0, int T) {
#pragma unroll
    for (int m = 0; m < L; ++m) {
        const int64_t o = base + (int64_t)min(t0 + m, T - 1) * rk;
        in.g[m] = g[o];
        in.q[m] = q[o];
        in.k[m] = k[o];
        in.b[m] = b[o];
    }
}

// ---------------------------------------------------------------------------------------
// Kernel 1: forward re-run in fp32 (one value-column slice per workgroup): the state entering
// every chunk, U = T (w.v - KG S), and (slice 0) T and P of every chunk
// ---------------------------------------------------------------------------------------
template <typename In, int DK, int DV, int DVS>
struct FwdCfg {
    static constexpr int TB = NT / DK, L = C / TB;
    static constexpr int KT = DK / 16, NCT = DVS / 16;
    static constexpr int NST = KT * NCT, SPW = (NST + 7) / 8;
    static constexpr int ES = (int)sizeof(In);
    static constexpr int LDF = DK + 4;        // fp32 [64][DK]
    static constexpr int LDT = DK + 16 / ES;  // In [64][DK]
    static constexpr int LDC = C + 4;
    static constexpr int LDV = DVS + 4;
    // operand tiles.  Pivoted chunk: KG = b.k.Gamma, KI = k / Gamma (then KR = KI.Gamma_C in
    // place), QG = q.Gamma.  Other chunk, while A and P are formed: G (fp32) and the raw k, b,
    // q; then KG and KR.
    static constexpr int KG = 0, KI = C * LDF * 4, QG = 2 * C * LDF * 4;
    static constexpr int GG = 0, RK = C * LDF * 4, RB = RK + C * LDT * ES, RQ = RB + C * LDT * ES;
    static constexpr int TILES = cmax(3 * C * LDF * 4, RQ + C * LDT * ES);
    static constexpr int AT = TILES;              // [64][LDC] A, then T in place
    static constexpr int WV = AT + C * LDC * 4;   // [64][LDV] w.v, then w.v - KG S
    static constexpr int UU = WV + C * LDV * 4;   // [64][LDV] U
    static constexpr int SC = UU + C * LDV * 4;   // [DK][LDV] S (operand copy)
    static constexpr int GC = SC + DK * LDV * 4;  // [DK] Gamma_C
    static constexpr int TOT = GC + DK * 4;       // [TB][DK] block sums of log alpha
    static constexpr int OFH = TOT + TB * DK * 4; // [TB][DK] sums over the earlier blocks, hi
    static constexpr int OFL = OFH + TB * DK * 4; // and lo
    static constexpr int FLG = OFL + TB * DK * 4;
    static constexpr int BYTES = FLG + 16;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(NT % DK == 0 && DVS % 16 == 0 && DV % DVS == 0, "shape");
};

template <typename In, int DK, int DV, int DVS>
__global__ __launch_bounds__(NT) void bwd_fwd_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ bgate, const In* __restrict__ wgate,
    const float* __restrict__ initial_state, float* __restrict__ s_ckpt, float* __restrict__ u_out,
    float* __restrict__ tp, int T, int H, int nslices) {
    using G = FwdCfg<In, DK, DV, DVS>;
    constexpr int TB = G::TB, L = G::L, KT = G::KT, NCT = G::NCT, NST = G::NST, SPW = G::SPW;
    constexpr int LDF = G::LDF, LDT = G::LDT, LDC = G::LDC, LDV = G::LDV;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    float* sKG = reinterpret_cast<float*>(smem + G::KG);
    float* sKI = reinterpret_cast<float*>(smem + G::KI);
    float* sQG = reinterpret_cast<float*>(smem + G::QG);
    float* sG = reinterpret_cast<float*>(smem + G::GG);
    In* sRK = reinterpret_cast<In*>(smem + G::RK);
    In* sRB = reinterpret_cast<In*>(smem + G::RB);
    In* sRQ = reinterpret_cast<In*>(smem + G::RQ);
    float* sAT = reinterpret_cast<float*>(smem + G::AT);
    float* sWV = reinterpret_cast<float*>(smem + G::WV);
    float* sUU = reinterpret_cast<float*>(smem + G::UU);
    float* sSC = reinterpret_cast<float*>(smem + G::SC);
    float* sGC = reinterpret_cast<float*>(smem + G::GC);
    float* sTOT = reinterpret_cast<float*>(smem + G::TOT);
    float* sOFH = reinterpret_cast<float*>(smem + G::OFH);
    float* sOFL = reinterpret_cast<float*>(smem + G::OFL);
    int* sFLG = reinterpret_cast<int*>(smem + G::FLG);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lane16 = lane & 15, grp4 = lane >> 4;
    const int bh = blockIdx.x / nslices, slice = blockIdx.x % nslices;
    const int bi = bh / H, h = bh % H, col0 = slice * DVS;
    const int nch = (T + C - 1) / C;
    const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;
    const int64_t base_k = ((int64_t)bi * T * H + h) * DK;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;

    f32x4 S[SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        S[s] = zero4();
        const int u = wave + 8 * s;
        if (initial_state && u < NST) {
            const int st = u % KT, ct = u / KT;
            const float* src = initial_state + ((int64_t)bh * DK + st * 16 + grp4 * 4) * DV + col0 + ct * 16 + lane16;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[s][r] = src[(int64_t)r * DV];
        }
    }
    // off-diagonal blocks of T: wave w < 6 forms block (LI, LJ) at level LI - LJ
    const int LI = wave < 3 ? wave + 1 : (wave < 5 ? wave - 1 : 3);
    const int LJ = wave < 3 ? wave : (wave < 5 ? wave - 3 : 0);

    const int ec_ = tid % DK, etb_ = tid / DK;
    // the next chunk's inputs are loaded one phase ahead (before the state update of the chunk
    // before it): key-side inputs, w and v of the slice
    constexpr int NWV = (C * DVS / 4 + NT - 1) / NT;  // groups of 4 value columns per thread
    KeyIn<In, L> in;
    Vec<In, 4> wr[NWV], vr[NWV];
    auto prefetch = [&](int nn) {
        const int tt0 = nn * C;
        load_key<In, L>(in, q, k, bgate, log_alpha, base_k + ec_, rk, tt0 + etb_ * L, T);
#pragma unroll
        for (int i = 0; i < NWV; ++i) {
            const int e = tid + i * NT, r = e / (DVS / 4), c4 = (e % (DVS / 4)) * 4;
            const int64_t o = base_v + (int64_t)min(tt0 + r, T - 1) * rv + col0 + c4;
            if (e < C * DVS / 4) {
                wr[i] = load_vec<In, 4>(wgate + o);
                vr[i] = load_vec<In, 4>(v + o);
            }
        }
    };
    prefetch(0);
    for (int n = 0; n < nch; ++n) {
        const int l16 = opq(lane16), g4 = opq(grp4), ec = opq(ec_), etb = opq(etb_);
        const int t0 = n * C;
        float* tpn = tp + ((int64_t)bh * nch + n) * 2 * C * C;
        // the state entering the chunk: checkpoint and operand copy
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int u = wave + 8 * s;
            if (u < NST) {
                const int st = u % KT, ct = u / KT;
                float* dst = s_ckpt + (((int64_t)bh * nch + n) * DK + st * 16 + g4 * 4) * DV + col0 + ct * 16 + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dst[(int64_t)r * DV] = S[s][r];
                    sSC[(st * 16 + g4 * 4 + r) * LDV + ct * 16 + l16] = S[s][r];
                }
            }
        }
        if (tid == 0) *sFLG = 0;
        // element phase, pass 1 (inputs prefetched): cumulative log-decay within the token block;
        // w.v of the slice
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
                const int e = tid + i * NT, r = e / (DVS / 4), c4 = (e % (DVS / 4)) * 4;
                if (e < C * DVS / 4) {
                    f32x4 wv = zero4();
                    if (t0 + r < T) {
#pragma unroll
                        for (int z = 0; z < 4; ++z) wv[z] = to_f32(wr[i].v[z]) * to_f32(vr[i].v[z]);
                    }
                    *reinterpret_cast<f32x4*>(sWV + r * LDV + c4) = wv;
                }
            }
        }
        lds_barrier();
        float off = 0.f, tot = 0.f, after = 0.f, oh = 0.f, ol = 0.f;
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
        const float run = sTOT[etb * DK + ec];
        sOFH[etb * DK + ec] = oh;
        sOFL[etb * DK + ec] = ol;
        if (etb == 0) {
            sGC[ec] = exp_any(tot);
            if (!(tot >= kMildLog)) *sFLG = 1;
        }
        lds_barrier();
        const bool mild = *sFLG == 0;
        // element phase, pass 2: operand tiles
#pragma unroll
        for (int m = 0; m < L; ++m) {
            const int i = etb * L + m, t = t0 + i;
            In qv = from_f32<In>(0.f), kv = qv, bv = qv;
            if (t < T) {
                qv = in.q[m];
                kv = in.k[m];
                bv = in.b[m];
            }
            const float Gi = x[m] + off;
            if (mild) {
                const float ga = exp_any(Gi);
                sKG[i * LDF + ec] = to_f32(bv) * to_f32(kv) * ga;
                sKI[i * LDF + ec] = to_f32(kv) * exp_any(-Gi);
                sQG[i * LDF + ec] = to_f32(qv) * ga;
            } else {
                sG[i * LDF + ec] = x[m];  // block-local
                sRK[i * LDT + ec] = kv;
                sRB[i * LDT + ec] = bv;
                sRQ[i * LDT + ec] = qv;
            }
        }
        if (n + 1 < nch) prefetch(n + 1);
        lds_barrier();
        // A (strictly lower, into the A/T tile) and, in slice 0, P (lower, to tp)
        if (mild) {
            // lower 16 x 16 blocks (I >= J) in the order (0,0) (1,0) (1,1) (2,0) ...: blocks 0-9 of
            // A and, in slice 0, blocks 10-19 of P; wave w takes blocks w, w + 8, w + 16
            const int nt = slice == 0 ? 20 : 10;
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
                if (u >= nt) continue;
                int I, J;
                blk(u, I, J);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = I * 16 + g4 * 4 + r, j = J * 16 + l16;
                    if (u < 10) sAT[i * LDC + j] = j < i ? acc[t][r] : 0.f;
                    else tpn[C * C + i * C + j] = j <= i ? acc[t][r] : 0.f;
                }
            }
            if (slice == 0) {  // P above the diagonal blocks is zero
                for (int e = tid; e < C * C; e += NT) {
                    const int i = e / C, j = e % C;
                    if (j / 16 > i / 16) tpn[C * C + e] = 0.f;
                }
            }
        } else {
            const int i = tid & 63, jg = tid >> 6;
            const int bI = i / L;
            for (int j = jg; j < C; j += 8) {
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
                if (slice == 0) tpn[C * C + i * C + j] = p;
            }
        }
        lds_barrier();
        // KG and KR = k.Gamma_C / Gamma for the state products
#pragma unroll
        for (int m = 0; m < L; ++m) {
            const int i = etb * L + m, t = t0 + i;
            if (mild) {
                sKI[i * LDF + ec] *= sGC[ec];
            } else {
                float kv = 0.f, bv = 0.f;
                if (t < T) {  // reloaded: keeping the raw inputs live costs registers everywhere
                    const int64_t o = base_k + (int64_t)t * rk + ec;
                    kv = to_f32(k[o]);
                    bv = to_f32(bgate[o]);
                }
                const float Gi = x[m] + off;
                sKG[i * LDF + ec] = bv * kv * exp_any(Gi);
                sKI[i * LDF + ec] = kv * exp_any((run - x[m]) + after);
            }
        }
        // T = (I + A)^{-1}: diagonal blocks by forward substitution (column j on lane j of
        // wave I), in place
        if (wave < 4 && lane < 16) {
            float* Ab = sAT + wave * 16 * LDC + wave * 16;
            float xs[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) xs[i] = i == lane ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                const float xm = xs[m];
#pragma unroll
                for (int i = m + 1; i < 16; ++i) xs[i] -= Ab[i * LDC + m] * xm;
                // keep each step's loads in their step: hoisted, the 120 loads would need as
                // many registers
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Ab[i * LDC + lane] = xs[i];
        }
        lds_barrier();
        // off-diagonal blocks, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, level by level; every
        // wave first takes the blocks of A it needs, before the levels overwrite them
        float ap[3][4];
#pragma unroll
        for (int kb = 0; kb < 3; ++kb)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int K = LJ + kb;
                ap[kb][s4] = (wave < 6 && K < LI) ? sAT[(LI * 16 + l16) * LDC + K * 16 + g4 + 4 * s4] : 0.f;
            }
        lds_barrier();
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
            if (wave < 6 && LI - LJ == d) {
                f32x4 z = zero4();
#pragma unroll
                for (int kb = 0; kb < 3; ++kb) {
                    const int K = LJ + kb;
                    if (K < LI) {
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4)
                            z = mfma4(z, ap[kb][s4], sAT[(K * 16 + g4 + 4 * s4) * LDC + LJ * 16 + l16]);
                    }
                }
                f32x4 tij = zero4();
#pragma unroll
                for (int e = 0; e < 4; ++e) tij = mfma4(tij, sAT[(LI * 16 + l16) * LDC + LI * 16 + 4 * g4 + e], z[e]);
#pragma unroll
                for (int r = 0; r < 4; ++r) sAT[(LI * 16 + g4 * 4 + r) * LDC + LJ * 16 + l16] = -tij[r];
            }
            lds_barrier();
        }
        if (slice == 0) {
            for (int e = tid; e < C * C; e += NT) {
                const int i = e / C, j = e % C;
                tpn[e] = j <= i ? sAT[i * LDC + j] : 0.f;
            }
        }
        // w.v - KG S, in place
        for (int u = wave; u < 4 * NCT; u += 8) {
            const int it = u % 4, ct = u / 4;
            f32x4 acc = zero4();
            mm_split<4, DK>(acc, [&](int m, int kk) { return sKG[(it * 16 + m) * LDF + kk]; },
                            [&](int kk, int nn) { return sSC[kk * LDV + ct * 16 + nn]; }, l16, g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* p = sWV + (it * 16 + g4 * 4 + r) * LDV + ct * 16 + l16;
                *p -= acc[r];
            }
        }
        lds_barrier();
        // U = T (w.v - KG S)
        for (int u = wave; u < 4 * NCT; u += 8) {
            const int it = u % 4, ct = u / 4;
            f32x4 acc = zero4();
            // T is lower triangular: blocks 0..it of the contraction, as separate chains
            mm_tail64(acc, [&](int m, int kk) { return kk < it * 16 + 16 ? sAT[(it * 16 + m) * LDC + kk] : 0.f; },
                      [&](int kk, int nn) { return sWV[kk * LDV + ct * 16 + nn]; }, 0, l16, g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = it * 16 + g4 * 4 + r, t = t0 + i;
                sUU[i * LDV + ct * 16 + l16] = acc[r];
                if (t < T) u_out[base_v + (int64_t)t * rv + col0 + ct * 16 + l16] = acc[r];
            }
        }
        lds_barrier();
        // S <- Gamma_C S + KR^T U
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int u = wave + 8 * s;
            if (u < NST) {
                const int st = u % KT, ct = u / KT;
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = S[s][r] * sGC[st * 16 + g4 * 4 + r];
                mm_split<4, C>(acc, [&](int m, int kk) { return sKI[kk * LDF + st * 16 + m]; },
                               [&](int kk, int nn) { return sUU[kk * LDV + ct * 16 + nn]; }, l16, g4);
                S[s] = acc;
            }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------------------
// Kernel 2: reverse pass over the chunks for dS (one value-column slice per workgroup)
// ---------------------------------------------------------------------------------------
template <typename In, int DK, int DV, int DVS>
struct StateCfg {
    static constexpr int TB = NT / DK;       // token blocks of the element phase
    static constexpr int L = C / TB;         // tokens per block
    static constexpr int KT = DK / 16, NCT = DVS / 16;
    static constexpr int NST = KT * NCT;     // 16 x 16 tiles of the dS slice
    static constexpr int SPW = (NST + 7) / 8;
    static constexpr int LDF = DK + 4;       // fp32 [64][DK]
    static constexpr int LDC = C + 4;        // fp32 [64][64]
    static constexpr int LDV = DVS + 4;      // fp32 [*][DVS]
    // KR, P and T are dead once dR is formed; q.Gamma and b.k.Gamma take their place
    static constexpr int KR = 0;                         // [64][LDF] k.Gamma_C / Gamma
    static constexpr int PP = KR + C * LDF * 4;          // [64][LDC] P
    static constexpr int TT = PP + C * LDC * 4;          // [64][LDC] T
    static constexpr int QG = 0;                         // [64][LDF] q.Gamma
    static constexpr int KG = QG + C * LDF * 4;          // [64][LDF] b.k.Gamma
    static constexpr int DO = TT + C * LDC * 4;          // [64][LDV] dO slice
    static constexpr int DU = DO + C * LDV * 4;          // [64][LDV] dU
    static constexpr int DR = DU + C * LDV * 4;          // [64][LDV] dR
    static constexpr int DS = DR + C * LDV * 4;          // [DK][LDV] dS' (operand copy)
    static constexpr int GC = DS + DK * LDV * 4;         // [DK] Gamma_C
    static constexpr int TOT = GC + DK * 4;              // [TB][DK] block sums of log alpha
    static constexpr int BYTES = TOT + TB * DK * 4;
    static_assert(BYTES <= 163840, "LDS budget exceeded");
    static_assert(KG + C * LDF * 4 <= DO, "q.Gamma and b.k.Gamma do not fit over KR, P, T");
    static_assert(NT % DK == 0 && C % TB == 0 && DVS % 16 == 0 && DV % DVS == 0, "shape");
};

template <typename In, int DK, int DV, int DVS>
__global__ __launch_bounds__(NT) void bwd_state_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const float* __restrict__ log_alpha,
    const In* __restrict__ bgate, const float* __restrict__ d_o, const float* __restrict__ d_final,
    const float* __restrict__ tp, float* __restrict__ ds_ckpt, float* __restrict__ dr_out,
    float* __restrict__ d_initial, int T, int H, int nslices) {
    using G = StateCfg<In, DK, DV, DVS>;
    constexpr int TB = G::TB, L = G::L, KT = G::KT, NCT = G::NCT, NST = G::NST, SPW = G::SPW;
    constexpr int LDF = G::LDF, LDC = G::LDC, LDV = G::LDV;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    float* sQG = reinterpret_cast<float*>(smem + G::QG);
    float* sKG = reinterpret_cast<float*>(smem + G::KG);
    float* sKR = reinterpret_cast<float*>(smem + G::KR);
    float* sT = reinterpret_cast<float*>(smem + G::TT);
    float* sP = reinterpret_cast<float*>(smem + G::PP);
    float* sDO = reinterpret_cast<float*>(smem + G::DO);
    float* sDU = reinterpret_cast<float*>(smem + G::DU);
    float* sDR = reinterpret_cast<float*>(smem + G::DR);
    float* sDS = reinterpret_cast<float*>(smem + G::DS);
    float* sGC = reinterpret_cast<float*>(smem + G::GC);
    float* sTOT = reinterpret_cast<float*>(smem + G::TOT);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lane16 = lane & 15, grp4 = lane >> 4;
    const int bh = blockIdx.x / nslices, slice = blockIdx.x % nslices;
    const int bi = bh / H, h = bh % H, col0 = slice * DVS;
    const int nch = (T + C - 1) / C;
    const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;  // elements between tokens
    const int64_t base_k = ((int64_t)bi * T * H + h) * DK;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;

    // dS slice in accumulators: tile u = wave + 8 s has row tile u % KT, column tile u / KT;
    // lane (n, g) holds dS[16 st + 4 g + r][16 ct + n]
    f32x4 dS[SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        dS[s] = zero4();
        const int u = wave + 8 * s;
        if (d_final && u < NST) {
            const int st = u % KT, ct = u / KT;
            const float* src = d_final + ((int64_t)bh * DK + st * 16 + grp4 * 4) * DV + col0 + ct * 16 + lane16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[s][r] = src[(int64_t)r * DV];
        }
    }

    const int ec_ = tid % DK, etb_ = tid / DK;  // element phase: channel, token block
    // the next chunk's inputs are loaded one phase ahead (before the dS update of the chunk
    // before it): key-side inputs, T and P, the dO slice
    constexpr int NTP = 2 * C * C / 4 / NT;             // float4 of T and P per thread
    constexpr int NDO = (C * DVS / 4 + NT - 1) / NT;    // float4 of dO per thread
    KeyIn<In, L> in;
    f32x4 tpv[NTP], dov[NDO];
    auto prefetch_key = [&](int nn) {
        load_key<In, L>(in, q, k, bgate, log_alpha, base_k + ec_, rk, nn * C + etb_ * L, T);
    };
    auto prefetch_tp = [&](int nn) {
        const int tt0 = nn * C;
        const float* src = tp + ((int64_t)bh * nch + nn) * 2 * C * C;
#pragma unroll
        for (int i = 0; i < NTP; ++i) tpv[i] = *reinterpret_cast<const f32x4*>(src + (tid + i * NT) * 4);
#pragma unroll
        for (int i = 0; i < NDO; ++i) {
            const int e = tid + i * NT, r = e / (DVS / 4), c4 = (e % (DVS / 4)) * 4;
            const int t = min(tt0 + r, T - 1);
            dov[i] = e < C * DVS / 4 ? *reinterpret_cast<const f32x4*>(d_o + base_v + (int64_t)t * rv + col0 + c4)
                                     : zero4();
        }
    };
    prefetch_key(nch - 1);
    prefetch_tp(nch - 1);
    for (int n = nch - 1; n >= 0; --n) {
        const int l16 = opq(lane16), g4 = opq(grp4), ec = opq(ec_), etb = opq(etb_);
        const int t0 = n * C;
        // dS' of this chunk: checkpoint for kernel 3 and operand copy
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int u = wave + 8 * s;
            if (u < NST) {
                const int st = u % KT, ct = u / KT;
                float* dst = ds_ckpt + (((int64_t)bh * nch + n) * DK + st * 16 + g4 * 4) * DV + col0 + ct * 16 + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dst[(int64_t)r * DV] = dS[s][r];
                    sDS[(st * 16 + g4 * 4 + r) * LDV + ct * 16 + l16] = dS[s][r];
                }
            }
        }
        // element phase, pass 1: cumulative log-decay within the token block (inputs prefetched)
        float x[L];
        {
            float run = 0.f;
#pragma unroll
            for (int m = 0; m < L; ++m) {
                run += t0 + etb * L + m < T ? in.g[m] : 0.f;
                x[m] = run;
            }
            sTOT[etb * DK + ec] = run;
        }
        // T and P of the chunk, and the dO slice (prefetched)
        {
#pragma unroll
            for (int i = 0; i < NTP; ++i) {
                const int e = tid + i * NT;
                const int mat = e / (C * C / 4), r = (e / (C / 4)) % C, c4 = (e % (C / 4)) * 4;
                *reinterpret_cast<f32x4*>((mat ? sP : sT) + r * LDC + c4) = tpv[i];
            }
#pragma unroll
            for (int i = 0; i < NDO; ++i) {
                const int e = tid + i * NT, r = e / (DVS / 4), c4 = (e % (DVS / 4)) * 4;
                if (e < C * DVS / 4) *reinterpret_cast<f32x4*>(sDO + r * LDV + c4) = t0 + r < T ? dov[i] : zero4();
            }
        }
        if (n > 0) prefetch_tp(n - 1);
        lds_barrier();
        // element phase, pass 2: decayed operands (q.Gamma and b.k.Gamma stay in registers until
        // their place is free)
        float qg[L], kg[L];
        {
            float off = 0.f, tot = 0.f, after = 0.f;
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const float vj = sTOT[j * DK + ec];
                tot += vj;
                if (j < etb) off += vj;
                if (j > etb) after += vj;
            }
            const float run = sTOT[etb * DK + ec];
            if (etb == 0) sGC[ec] = exp_any(tot);
#pragma unroll
            for (int m = 0; m < L; ++m) {
                const int i = etb * L + m, t = t0 + i;
                float qv = 0.f, kv = 0.f, bv = 0.f;
                if (t < T) {
                    qv = to_f32(in.q[m]);
                    kv = to_f32(in.k[m]);
                    bv = to_f32(in.b[m]);
                }
                const float Gi = x[m] + off;
                const float ga = exp_any(Gi);
                qg[m] = qv * ga;
                kg[m] = bv * kv * ga;
                sKR[i * LDF + ec] = kv * exp_any((run - x[m]) + after);
            }
        }
        lds_barrier();
        // dU = P^T dO + KR dS'   (tile: token rows jt, value columns ct)
        for (int u = wave; u < 4 * NCT; u += 8) {
            const int jt = u % 4, ct = u / 4;
            f32x4 acc = zero4();
            mm_tail64(acc, [&](int m, int kk) { return sP[kk * LDC + jt * 16 + m]; },
                      [&](int kk, int nn) { return sDO[kk * LDV + ct * 16 + nn]; }, jt, l16, g4);
            mm_split<4, DK>(acc, [&](int m, int kk) { return sKR[(jt * 16 + m) * LDF + kk]; },
                            [&](int kk, int nn) { return sDS[kk * LDV + ct * 16 + nn]; }, l16, g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) sDU[(jt * 16 + g4 * 4 + r) * LDV + ct * 16 + l16] = acc[r];
        }
        lds_barrier();
        // dR = T^T dU
        for (int u = wave; u < 4 * NCT; u += 8) {
            const int it = u % 4, ct = u / 4;
            f32x4 acc = zero4();
            mm_tail64(acc, [&](int m, int kk) { return sT[kk * LDC + it * 16 + m]; },
                      [&](int kk, int nn) { return sDU[kk * LDV + ct * 16 + nn]; }, it, l16, g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = it * 16 + g4 * 4 + r, t = t0 + i;
                sDR[i * LDV + ct * 16 + l16] = acc[r];
                if (t < T) dr_out[base_v + (int64_t)t * rv + col0 + ct * 16 + l16] = acc[r];
            }
        }
        lds_barrier();
#pragma unroll
        for (int m = 0; m < L; ++m) {
            const int i = etb * L + m;
            sQG[i * LDF + ec] = qg[m];
            sKG[i * LDF + ec] = kg[m];
        }
        lds_barrier();
        // the next chunk's key-side inputs: issued here, their registers are live only across
        // this phase (earlier, they force spills, and a spill reload would wait behind them)
        if (n > 0) prefetch_key(n - 1);
        // dS = Gamma_C dS' + QG^T dO - KG^T dR
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int u = wave + 8 * s;
            if (u < NST) {
                const int st = u % KT, ct = u / KT;
                f32x4 acc2[2] = {zero4(), zero4()};
                mm_n<2, C>(acc2, [&](int t, int m, int kk) { return (t ? sKG : sQG)[kk * LDF + st * 16 + m]; },
                           [&](int t, int kk, int nn) { return (t ? sDR : sDO)[kk * LDV + ct * 16 + nn]; }, l16, g4);
#pragma unroll
                for (int r = 0; r < 4; ++r) dS[s][r] = dS[s][r] * sGC[st * 16 + g4 * 4 + r] + acc2[0][r] - acc2[1][r];
            }
        }
        lds_barrier();
    }
    if (d_initial) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int u = wave + 8 * s;
            if (u < NST) {
                const int st = u % KT, ct = u / KT;
                float* dst = d_initial + ((int64_t)bh * DK + st * 16 + grp4 * 4) * DV + col0 + ct * 16 + lane16;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)r * DV] = dS[s][r];
            }
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
    // region 1: dO, dR, U (phases 1-2); then G and the raw q, k, b (phases 3-5)
    static constexpr int DO = 0, DR = C * LDV * 4, UU = 2 * C * LDV * 4;
    static constexpr int GG = 0, QQ = C * LDF * 4, KK = QQ + C * LDT * ES, BB = KK + C * LDT * ES;
    static constexpr int R1 = cmax(3 * C * LDV * 4, BB + C * LDT * ES);
    // region 2: a half of S or dS' (phase 2); then dA, dP (phases 3-4); then dG (phase 5)
    static constexpr int SH = R1, DA = R1, DP = R1 + C * LDC * 4, DG = R1;
    static constexpr int R2 = cmax(DK * LDH * 4, cmax(2 * C * LDC * 4, C * LDF * 4));
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
    float* __restrict__ dw, int T, int H) {
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

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int nch = (T + C - 1) / C;
    const int n = blockIdx.x % nch, bh = blockIdx.x / nch;
    const int bi = bh / H, h = bh % H, t0 = n * C;
    const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;
    const int64_t base_k = ((int64_t)bi * T * H + h) * DK;
    const int64_t base_v = ((int64_t)bi * T * H + h) * DV;
    const float* Sg = s_ckpt + ((int64_t)bh * nch + n) * DK * DV;
    const float* dSg = ds_ckpt + ((int64_t)bh * nch + n) * DK * DV;

    // this wave's output tiles: channel column tile ct, token row tiles it0 + ITS j
    const int ct = wave % KT, it0 = wave / KT;
    const int c = ct * 16 + l16;  // the channel of this lane's accumulator column

    if (tid < DK) {
        sXD[tid] = 0.f;
        sXR[tid] = 0.f;
    }
    if (tid == 0) *sFLG = 0;

    // ---- phase 1: dO, dR, U of the chunk; dv = dR.w, dw = dR.v ----
    for (int e = tid; e < C * DV / 4; e += NT) {
        const int r = e / (DV / 4), c4 = (e % (DV / 4)) * 4, t = t0 + r;
        f32x4 o4 = zero4(), r4 = zero4(), u4 = zero4();
        if (t < T) {
            const int64_t off = base_v + (int64_t)t * rv + c4;
            o4 = *reinterpret_cast<const f32x4*>(d_o + off);
            r4 = *reinterpret_cast<const f32x4*>(dr_in + off);
            u4 = *reinterpret_cast<const f32x4*>(u_in + off);
            const Vec<In, 4> w4 = load_vec<In, 4>(wgate + off), v4 = load_vec<In, 4>(v + off);
            f32x4 a4, b4;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                a4[x] = r4[x] * to_f32(w4.v[x]);
                b4[x] = r4[x] * to_f32(v4.v[x]);
            }
            *reinterpret_cast<f32x4*>(dv + off) = a4;
            *reinterpret_cast<f32x4*>(dw + off) = b4;
        }
        *reinterpret_cast<f32x4*>(sDO + r * LDV + c4) = o4;
        *reinterpret_cast<f32x4*>(sDR + r * LDV + c4) = r4;
        *reinterpret_cast<f32x4*>(sU + r * LDV + c4) = u4;
    }

    // ---- phase 2: X1 = dO S^T, X2 = dR S^T, X3 = U dS'^T over two halves of the value axis ----
    f32x4 X1[TPW], X2[TPW], X3[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) X1[j] = X2[j] = X3[j] = zero4();
    constexpr int HV = DV / 2;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        __syncthreads();
        for (int e = tid; e < DK * HV / 4; e += NT) {
            const int r = e / (HV / 4), c4 = (e % (HV / 4)) * 4;
            *reinterpret_cast<f32x4*>(sSH + r * LDH + c4) = *reinterpret_cast<const f32x4*>(Sg + r * DV + hh * HV + c4);
        }
        __syncthreads();
        {
            f32x4 acc[2 * TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                acc[j] = X1[j];
                acc[TPW + j] = X2[j];
            }
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
        __syncthreads();
        for (int e = tid; e < DK * HV / 4; e += NT) {
            const int r = e / (HV / 4), c4 = (e % (HV / 4)) * 4;
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dSg + r * DV + hh * HV + c4);
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sg + r * DV + hh * HV + c4);
            *reinterpret_cast<f32x4*>(sSH + r * LDH + c4) = d4;
            atomicAdd(sXD + r, d4[0] * s4[0] + d4[1] * s4[1] + d4[2] * s4[2] + d4[3] * s4[3]);
        }
        __syncthreads();
        mm_n<TPW, HV>(X3, [&](int t, int m, int kk) { return sU[((it0 + ITS * t) * 16 + m) * LDV + hh * HV + kk]; },
                      [&](int, int kk, int nn) { return sSH[(ct * 16 + nn) * LDH + kk]; }, l16, g4);
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) X2[j] = -X2[j];  // -dR S^T
    __syncthreads();

    // ---- phase 3: dA = -dR U^T (j < i), dP = dO U^T (j <= i); zero above the diagonal ----
    {
        // wave w: block pairs p = w and w + 8, (I, J) = (p / 4, p % 4), both dA and dP
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
    __syncthreads();  // region 1 (dO, dR, U) is free from here on

    // element phase: G (chunk-local cumulative log alpha) and the raw q, k, b of the chunk
    const int ec = tid % DK, etb = tid / DK;
    {
        KeyIn<In, L> in;
        load_key<In, L>(in, q, k, bgate, log_alpha, base_k + ec, rk, t0 + etb * L, T);
        float x[L];
        float run = 0.f;
#pragma unroll
        for (int m = 0; m < L; ++m) {
            run += t0 + etb * L + m < T ? in.g[m] : 0.f;
            x[m] = run;
        }
        sTOT[etb * DK + ec] = run;
        __syncthreads();
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
            if (t < T) {
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
    __syncthreads();
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
#pragma unroll
        for (int kb = 0; kb < C; kb += 4) {
            const int r = kb + g4;  // contraction token of this lane group
            const float Gr = Gof(r, c);
            const float kr = to_f32(sK[r * LDT + c]);
            const float ep = exp_any(Gr), en = exp_any(-Gr);
            const float ki = kr * en;                        // k / Gamma
            const float kg = to_f32(sB[r * LDT + c]) * kr * ep;  // kh.Gamma
            const float qg = to_f32(sQ[r * LDT + c]) * ep;       // q.Gamma
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int it = it0 + ITS * j;
                if (kb < it * 16 + 16) {
                    X1[j] = mfma4(X1[j], sDP[(it * 16 + l16) * LDC + r], ki);
                    X2[j] = mfma4(X2[j], sDA[(it * 16 + l16) * LDC + r], ki);
                }
                if (kb + 4 > it * 16) {
                    X3[j] = mfma4(X3[j], sDA[r * LDC + it * 16 + l16], kg);
                    X3[j] = mfma4(X3[j], sDP[r * LDC + it * 16 + l16], qg);
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
                for (int jj = 0; jj <= i; ++jj) {
                    const float f = exp_any(Gdiff(i, jj, c)) * to_f32(sK[jj * LDT + c]);
                    sq += sDP[i * LDC + jj] * f;
                    sh += sDA[i * LDC + jj] * f;
                }
                for (int ii = i; ii < C; ++ii) {
                    const float f = exp_any(Gdiff(ii, i, c));
                    const float kh = to_f32(sB[ii * LDT + c]) * to_f32(sK[ii * LDT + c]);
                    sk += (sDA[ii * LDC + i] * kh + sDP[ii * LDC + i] * to_f32(sQ[ii * LDT + c])) * f;
                }
                const float ep = exp_any(Gof(i, c));
                X1[j][r] = ep * X1[j][r] + sq;
                X2[j][r] = ep * X2[j][r] + sh;
                X3[j][r] = exp_any(Gsuf(i, c)) * X3[j][r] + sk;
            }
        }
    }
    __syncthreads();  // dA, dP are consumed: region 2 takes dG

    // ---- phase 5: dq, dk, db; the per-token decay gradient dG ----
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int it = it0 + ITS * j;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = it * 16 + g4 * 4 + r, t = t0 + i;
            const float qv = to_f32(sQ[i * LDT + c]), kv = to_f32(sK[i * LDT + c]), bv = to_f32(sB[i * LDT + c]);
            const float dqv = X1[j][r], dkh = X2[j][r];
            const float dkv = X3[j][r] + bv * dkh;
            sDG[i * LDF + c] = qv * dqv + 2.f * bv * kv * dkh - kv * dkv;
            if (t < T) {
                const int64_t o = base_k + (int64_t)t * rk + c;
                dq[o] = dqv;
                dk[o] = dkv;
                db[o] = kv * dkh;
            }
        }
    }
    __syncthreads();
    // reverse cumulative sum over the chunk, plus the G_C terms
    {
        float run = 0.f;
#pragma unroll
        for (int m = L - 1; m >= 0; --m) run += sDG[(etb * L + m) * LDF + ec];
        sTOT[etb * DK + ec] = run;
        __syncthreads();
        float after = sXR[ec] + sGC[ec] * sXD[ec];
#pragma unroll
        for (int j = 0; j < TB; ++j)
            if (j > etb) after += sTOT[j * DK + ec];
        run = after;
#pragma unroll
        for (int m = L - 1; m >= 0; --m) {
            const int i = etb * L + m, t = t0 + i;
            run += sDG[i * LDF + ec];
            if (t < T) dg[base_k + (int64_t)t * rk + ec] = run;
        }
    }
}

template <typename In, int D, int DVS>
hipError_t launch_state(const BwdArgs& a, int nslices) {
    hipLaunchKernelGGL((bwd_state_kernel<In, D, D, DVS>), dim3((unsigned)(a.B * a.H * nslices)), dim3(NT), 0,
                       (hipStream_t)a.stream, (const In*)a.q, (const In*)a.k, a.log_alpha, (const In*)a.b,
                       a.d_o, a.d_final_state, a.tp, a.ds_ckpt, a.dr, a.g_s0, (int)a.T, (int)a.H, nslices);
    return hipGetLastError();
}

template <typename In, int D>
hipError_t launch_grad(const BwdArgs& a) {
    const int64_t nch = (a.T + C - 1) / C;
    hipLaunchKernelGGL((bwd_chunk_kernel<In, D, D>), dim3((unsigned)(a.B * a.H * nch)), dim3(NT), 0,
                       (hipStream_t)a.stream, (const In*)a.q, (const In*)a.k, (const In*)a.v, a.log_alpha,
                       (const In*)a.b, (const In*)a.w, a.d_o, a.s_ckpt, a.ds_ckpt, a.u, a.dr, a.g_q, a.g_k,
                       a.g_v, a.g_log_alpha, a.g_b, a.g_w, (int)a.T, (int)a.H);
    return hipGetLastError();
}

template <typename In, int D, int DVS>
hipError_t launch_fwd(const BwdArgs& a, int nslices) {
    hipLaunchKernelGGL((bwd_fwd_kernel<In, D, D, DVS>), dim3((unsigned)(a.B * a.H * nslices)), dim3(NT), 0,
                       (hipStream_t)a.stream, (const In*)a.q, (const In*)a.k, (const In*)a.v, a.log_alpha,
                       (const In*)a.b, (const In*)a.w, a.initial_state, a.s_ckpt, a.u, a.tp, (int)a.T, (int)a.H,
                       nslices);
    return hipGetLastError();
}

template <typename In, int D>
hipError_t launch_bwd_typed(const BwdArgs& a) {
    // forward re-run: at most 32 value columns per workgroup at d = 128 (LDS)
    hipError_t e;
    const int64_t bh = a.B * a.H;
    if (D == 64 && bh >= a.cus) e = launch_fwd<In, D, (D == 64 ? 64 : 32)>(a, D / (D == 64 ? 64 : 32));
    else if (bh * (D / 32) >= a.cus) e = launch_fwd<In, D, 32>(a, D / 32);
    else e = launch_fwd<In, D, 16>(a, D / 16);
    if (e != hipSuccess) return e;
    // reverse pass: the widest value slice (at most 64 columns) that still gives at least one
    // workgroup per compute unit, else 16 columns
    if (bh * (D / 64) >= a.cus) e = launch_state<In, D, 64>(a, D / 64);
    else if (bh * (D / 32) >= a.cus) e = launch_state<In, D, 32>(a, D / 32);
    else e = launch_state<In, D, 16>(a, D / 16);
    if (e != hipSuccess) return e;
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
