// gdn2_mixer.hip -- the elementwise steps on either side of the recurrence, each fused into
// one pass over HBM (page "Why NVIDIA Gated DeltaNet-2 separates erase and write gates",
// axbrief.com: the layer's architecture -- query and key through a short causal convolution,
// SiLU and L2 normalisation, value through the convolution and SiLU, the output through RMS
// normalisation and a SiLU output gate; section "Gated Delta Rule-2": the erase and write
// gates are sigmoids of projections of the token).
//
//   prep: from the projections' outputs xq, xk, xv, xb, xw, xa to the recurrence's inputs
//         q = L2(SiLU(conv(xq))), k = L2(SiLU(conv(xk))), v = SiLU(conv(xv)),
//         b = sigmoid(xb), w = sigmoid(xw), log alpha = log sigmoid(xa);
//   out:  y = o / sqrt(mean(o^2) + eps) * gamma * SiLU(z).
// The convolution is depthwise and causal with 4 taps: tap j of a channel multiplies its input
// at token t - 3 + j, and tokens before the start of the sequence are zero.
//
// prep: eight key and eight value channels per lane, a head per D / 8 lanes, a run of
// consecutive tokens per wave with the convolution window in registers; the L2 norms of q and
// k are reductions over a head's lanes (no LDS, no barrier).  out: rows of
// dv fp32 values, four per lane (16-byte loads), two rows per wave at dv = 128.
#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {
namespace mix {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int NTW = 16;  // consecutive tokens per prep workgroup

constexpr float kLn2 = 0.6931471805599453f;

// The activations use the hardware base-2 exponential and logarithm and the hardware
// reciprocal (about 1 ulp each; the sigmoid is gdn2_device.h's); these passes are limited by
// vector ALU issue, not by HBM, once IEEE division and a library log1p are in them.
__device__ __forceinline__ float log_sigmoid_f(float x) {
    // min(x, 0) - log(1 + e), e = e^-|x| in (0, 1]; log(1 + e) by its series below 2^-7
    // (three terms, error < e^4 / 4), else through the hardware logarithm
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float l = e < 0.0078125f ? e * (1.f - e * (0.5f - e * (1.f / 3.f)))
                                   : __builtin_amdgcn_logf(1.f + e) * kLn2;
    return fminf(x, 0.f) - l;
}
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// wave-wide sum over lanes [base, base + width) with width a power of two <= 64
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename In, int N>
__device__ __forceinline__ void store_n(In* p, const float (&x)[N]) {
    if constexpr (N == 1) {
        *p = from_f32<In>(x[0]);
    } else {
        typedef In V __attribute__((ext_vector_type(N)));
        V v;
#pragma unroll
        for (int e = 0; e < N; ++e) v[e] = from_f32<In>(x[e]);
        *reinterpret_cast<V*>(p) = v;
    }
}

// Eight channels per lane (16-byte bf16 accesses): a head's D channels take D / 8 lanes, so a
// wave holds 64 * 8 / D heads.  A workgroup has three waves for the same heads and the same
// run of NTW consecutive tokens: wave 0 makes q (and b), wave 1 k (and log alpha), wave 2 v
// (and w).  Each walks the run with its four taps per channel and the last three convolution
// inputs in registers, so every input row is read once, plus three rows before the run; the
// L2 norms are reductions over a head's lanes (no LDS, no barrier).
// GATES false: q, k and v only (the gates are activated inside the recurrence kernel).
template <typename In, int DK, int DV, bool GATES>
__global__ __launch_bounds__(192) void prep_kernel(
    const In* __restrict__ xq, const In* __restrict__ xk, const In* __restrict__ xv,
    const In* __restrict__ xb, const In* __restrict__ xw, const In* __restrict__ xa,
    const float* __restrict__ cq, const float* __restrict__ ck, const float* __restrict__ cv,
    In* __restrict__ q, In* __restrict__ k, In* __restrict__ v, In* __restrict__ b, In* __restrict__ w,
    float* __restrict__ log_alpha, int T, int H, int nrun, int nhg, float eps) {
    static_assert(DK == DV, "one head per lane group");
    constexpr int CH = 8, LPH = DK / CH;  // channels per lane, lanes per head
    constexpr int HPW = 64 / LPH;         // heads per wave
    const int role = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = blockIdx.x % nhg, rest = blockIdx.x / nhg;
    const int t0 = (rest % nrun) * NTW, bi = rest / nrun;
    const int h = g * HPW + lane / LPH;
    const bool live = h < H;
    const int c0 = (lane % LPH) * CH;
    const int hs = live ? h : 0;
    const int64_t st = (int64_t)H * DK;  // token stride (dk = dv)
    const int64_t off0 = (((int64_t)bi * T + t0) * H + hs) * DK + c0;
    const In* x = role == 0 ? xq : (role == 1 ? xk : xv);
    const In* gx = role == 0 ? xb : (role == 1 ? xa : xw);
    const float* cw = role == 0 ? cq : (role == 1 ? ck : cv);
    In* dst = role == 0 ? q : (role == 1 ? k : v);
    In* gdst = role == 0 ? b : w;
    float tw[CH][4];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(cw + (int64_t)(hs * DK + c0 + e) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) tw[e][j] = a[j];
    }
    float win[3][CH];  // inputs at t - 3, t - 2, t - 1
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int tt = t0 - 3 + j;
        if (tt >= 0) {
            const Vec<In, CH> r = load_vec<In, CH>(x + off0 + (int64_t)(j - 3) * st);
#pragma unroll
            for (int e = 0; e < CH; ++e) win[j][e] = to_f32(r.v[e]);
        } else {
#pragma unroll
            for (int e = 0; e < CH; ++e) win[j][e] = 0.f;
        }
    }
    const int nt = min(NTW, T - t0);
    // a full run is unrolled in groups of four tokens whose loads are issued together
    constexpr int G4 = 4;
    for (int i0 = 0; i0 < nt; i0 += G4) {
        Vec<In, CH> rs[G4], grs[G4];
#pragma unroll
        for (int d = 0; d < G4; ++d) {
            const int64_t off = off0 + (int64_t)min(i0 + d, nt - 1) * st;
            rs[d] = load_vec<In, CH>(x + off);
            if constexpr (GATES) grs[d] = load_vec<In, CH>(gx + off);
        }
#pragma unroll
        for (int d = 0; d < G4; ++d) {
        const int i = i0 + d;
        if (i >= nt) break;
        const int64_t off = off0 + (int64_t)i * st;
        const Vec<In, CH>& r = rs[d];
        const Vec<In, CH>& gr = grs[d];
        float u[CH], ss = 0.f;
#pragma unroll
        for (int e = 0; e < CH; ++e) {
            const float cur = to_f32(r.v[e]);
            u[e] = silu_f(tw[e][0] * win[0][e] + tw[e][1] * win[1][e] + tw[e][2] * win[2][e] + tw[e][3] * cur);
            win[0][e] = win[1][e];
            win[1][e] = win[2][e];
            win[2][e] = cur;
            ss += u[e] * u[e];
        }
        float gv[CH];
        if constexpr (GATES) {
            if (role == 1) {
#pragma unroll
                for (int e = 0; e < CH; ++e) gv[e] = log_sigmoid_f(to_f32(gr.v[e]));
            } else {
#pragma unroll
                for (int e = 0; e < CH; ++e) gv[e] = sigmoid_f(to_f32(gr.v[e]));
            }
        }
        if (role < 2) {  // q, k: L2 normalisation over the head
            ss = group_sum<LPH>(ss);
            const float inv = __builtin_amdgcn_rsqf(ss + eps);  // hardware 1/sqrt (about 1 ulp)
#pragma unroll
            for (int e = 0; e < CH; ++e) u[e] *= inv;
        }
        if (live) {
            store_n<In, CH>(dst + off, u);
            if constexpr (GATES) {
                if (role == 1) store_n<float, CH>(log_alpha + off, gv);
                else store_n<In, CH>(gdst + off, gv);
            }
        }
        }
    }
}

// RPW rows per wave (64 / RPW lanes per row), EL = DV * RPW / 64 elements per lane
template <typename OT, typename In, int DV>
__global__ __launch_bounds__(256) void out_kernel(const OT* __restrict__ o, const In* __restrict__ z,
                                                  const float* __restrict__ gamma, In* __restrict__ y,
                                                  int64_t rows, float eps) {
    constexpr int EL = 4, LPR = DV / EL, RPW = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const int c0 = (lane % LPR) * EL;
    const bool live = row < rows;
    const int64_t off = (live ? row : 0) * DV + c0;
    const Vec<OT, EL> ov = load_vec<OT, EL>(o + off);
    const Vec<In, EL> zv = load_vec<In, EL>(z + off);
    const f32x4 g = *reinterpret_cast<const f32x4*>(gamma + c0);
    float x[EL], s = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
        x[e] = to_f32(ov.v[e]);
        s += x[e] * x[e];
    }
    s = group_sum<LPR>(s);
    const float inv = __builtin_amdgcn_rsqf(s * (1.f / DV) + eps);  // hardware 1/sqrt (about 1 ulp)
    float r[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) r[e] = x[e] * inv * g[e] * silu_f(to_f32(zv.v[e]));
    if (live) store_n<In, EL>(y + off, r);
}

template <typename In, int D>
hipError_t launch_prep_t(const MixerPrepArgs& a) {
    constexpr int HPW = 64 / (D / 8);  // heads per wave
    const int nrun = (int)((a.T + NTW - 1) / NTW);  // workgroups along the tokens
    const int nhg = (int)((a.H + HPW - 1) / HPW);
    auto kern = a.b ? prep_kernel<In, D, D, true> : prep_kernel<In, D, D, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.B * nrun * nhg)), dim3(192), 0, (hipStream_t)a.stream, (const In*)a.xq, (const In*)a.xk, (const In*)a.xv, (const In*)a.xb,
                       (const In*)a.xw, (const In*)a.xa, a.conv_q, a.conv_k, a.conv_v, (In*)a.q, (In*)a.k, (In*)a.v,
                       (In*)a.b, (In*)a.w, a.log_alpha, (int)a.T, (int)a.H, nrun, nhg, a.eps);
    return hipGetLastError();
}

template <typename OT, typename In, int D>
hipError_t launch_out_t(const MixerOutArgs& a) {
    const int64_t rows = a.B * a.T * a.H;
    constexpr int RPW = 64 / (D / 4);  // rows per wave
    const int64_t rows_per_group = 4 * RPW;
    hipLaunchKernelGGL((out_kernel<OT, In, D>), dim3((unsigned)((rows + rows_per_group - 1) / rows_per_group)),
                       dim3(256), 0, (hipStream_t)a.stream, (const OT*)a.o, (const In*)a.z, a.gamma, (In*)a.y,
                       rows, a.eps);
    return hipGetLastError();
}

}  // namespace mix

hipError_t launch_mixer_prep(const MixerPrepArgs& a) {
    if (a.dk != a.dv) return hipErrorInvalidValue;
    if (a.dtype_bf16) {
        if (a.dk == 128) return mix::launch_prep_t<bf16, 128>(a);
        if (a.dk == 64) return mix::launch_prep_t<bf16, 64>(a);
    } else {
        if (a.dk == 128) return mix::launch_prep_t<float, 128>(a);
        if (a.dk == 64) return mix::launch_prep_t<float, 64>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mixer_out(const MixerOutArgs& a) {
    if (a.dtype_bf16) {
        if (a.o_f32) {
            if (a.dv == 128) return mix::launch_out_t<float, bf16, 128>(a);
            if (a.dv == 64) return mix::launch_out_t<float, bf16, 64>(a);
        } else {
            if (a.dv == 128) return mix::launch_out_t<bf16, bf16, 128>(a);
            if (a.dv == 64) return mix::launch_out_t<bf16, bf16, 64>(a);
        }
    } else {
        if (a.dv == 128) return mix::launch_out_t<float, float, 128>(a);
        if (a.dv == 64) return mix::launch_out_t<float, float, 64>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn2
