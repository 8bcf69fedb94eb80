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
// prep: one workgroup per (sequence, head, block of 64 tokens) with DK + DV threads; thread c <
// DK owns key channel c (q, k, b, log alpha), the others own value channels (v, w).  Each
// thread walks the block's tokens with the last three convolution inputs in registers, so
// every input element is read once (plus three tokens before the block).  SiLU(conv) of q and
// k goes to LDS; one wave per (token, q or k) row forms its norm; the key threads then scale
// and store.  out: one wave per (token, head) row.
#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {
namespace mix {

constexpr int TBK = 64;  // tokens per prep workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sigmoid_f(float x) {
    // 1 / (1 + e^-x) without overflow: e^-|x| <= 1
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float r = 1.f / (1.f + e);
    return x >= 0.f ? r : e * r;
}
__device__ __forceinline__ float log_sigmoid_f(float x) {
    // min(x, 0) - log(1 + e^-|x|)
    return fminf(x, 0.f) - log1pf(__builtin_amdgcn_exp2f(-fabsf(x) * kLog2e));
}
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename In, int DK, int DV>
__global__ __launch_bounds__(DK + DV) void prep_kernel(
    const In* __restrict__ xq, const In* __restrict__ xk, const In* __restrict__ xv,
    const In* __restrict__ xb, const In* __restrict__ xw, const In* __restrict__ xa,
    const float* __restrict__ cq, const float* __restrict__ ck, const float* __restrict__ cv,
    In* __restrict__ q, In* __restrict__ k, In* __restrict__ v, In* __restrict__ b, In* __restrict__ w,
    float* __restrict__ log_alpha, int T, int H, int nblk, float eps) {
    constexpr int NTH = DK + DV;
    __shared__ float sU[2][TBK][DK];  // SiLU(conv) of q and k
    __shared__ float sInv[2][TBK];    // 1 / sqrt(sum of squares + eps)
    const int tid = threadIdx.x;
    const int blk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
    const int bi = bh / H, h = bh % H;
    const int t0 = blk * TBK;
    const int nt = min(TBK, T - t0);
    const bool key = tid < DK;
    const int c = key ? tid : tid - DK;
    const int D = key ? DK : DV;
    // element (t, h, c) of sequence bi: ((bi * T + t) * H + h) * D + c
    const int64_t base = ((int64_t)bi * T * H + h) * D + c;
    const int64_t stride = (int64_t)H * D;

    if (key) {
        const f32x4 wq = *reinterpret_cast<const f32x4*>(cq + (int64_t)(h * DK + c) * 4);
        const f32x4 wk = *reinterpret_cast<const f32x4*>(ck + (int64_t)(h * DK + c) * 4);
        float q1 = 0.f, q2 = 0.f, q3 = 0.f, k1 = 0.f, k2 = 0.f, k3 = 0.f;  // inputs at t-1, t-2, t-3
        if (t0 >= 3) {
            q3 = to_f32(xq[base + (t0 - 3) * stride]);
            k3 = to_f32(xk[base + (t0 - 3) * stride]);
        }
        if (t0 >= 2) {
            q2 = to_f32(xq[base + (t0 - 2) * stride]);
            k2 = to_f32(xk[base + (t0 - 2) * stride]);
        }
        if (t0 >= 1) {
            q1 = to_f32(xq[base + (t0 - 1) * stride]);
            k1 = to_f32(xk[base + (t0 - 1) * stride]);
        }
        for (int i = 0; i < nt; ++i) {
            const int64_t o = base + (t0 + i) * stride;
            const float xq0 = to_f32(xq[o]), xk0 = to_f32(xk[o]);
            const float yq = wq[0] * q3 + wq[1] * q2 + wq[2] * q1 + wq[3] * xq0;
            const float yk = wk[0] * k3 + wk[1] * k2 + wk[2] * k1 + wk[3] * xk0;
            sU[0][i][c] = silu_f(yq);
            sU[1][i][c] = silu_f(yk);
            q3 = q2; q2 = q1; q1 = xq0;
            k3 = k2; k2 = k1; k1 = xk0;
            b[o] = from_f32<In>(sigmoid_f(to_f32(xb[o])));
            log_alpha[o] = log_sigmoid_f(to_f32(xa[o]));
        }
    } else {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(cv + (int64_t)(h * DV + c) * 4);
        float v1 = 0.f, v2 = 0.f, v3 = 0.f;
        if (t0 >= 3) v3 = to_f32(xv[base + (t0 - 3) * stride]);
        if (t0 >= 2) v2 = to_f32(xv[base + (t0 - 2) * stride]);
        if (t0 >= 1) v1 = to_f32(xv[base + (t0 - 1) * stride]);
        for (int i = 0; i < nt; ++i) {
            const int64_t o = base + (t0 + i) * stride;
            const float xv0 = to_f32(xv[o]);
            const float yv = wv[0] * v3 + wv[1] * v2 + wv[2] * v1 + wv[3] * xv0;
            v3 = v2; v2 = v1; v1 = xv0;
            v[o] = from_f32<In>(silu_f(yv));
            w[o] = from_f32<In>(sigmoid_f(to_f32(xw[o])));
        }
    }
    __syncthreads();
    // norms: one wave per (q or k, token) row
    constexpr int NW = NTH / 64;
    const int wave = tid >> 6, lane = tid & 63;
    for (int row = wave; row < 2 * nt; row += NW) {
        const int which = row / nt, i = row % nt;
        float s = 0.f;
#pragma unroll
        for (int cc = lane; cc < DK; cc += 64) {
            const float u = sU[which][i][cc];
            s += u * u;
        }
        s = wave_sum(s);
        if (lane == 0) sInv[which][i] = 1.f / sqrtf(s + eps);
    }
    __syncthreads();
    if (key) {
        for (int i = 0; i < nt; ++i) {
            const int64_t o = base + (t0 + i) * stride;
            q[o] = from_f32<In>(sU[0][i][c] * sInv[0][i]);
            k[o] = from_f32<In>(sU[1][i][c] * sInv[1][i]);
        }
    }
}

template <typename OT, typename In, int DV>
__global__ __launch_bounds__(256) void out_kernel(const OT* __restrict__ o, const In* __restrict__ z,
                                                  const float* __restrict__ gamma, In* __restrict__ y,
                                                  int64_t rows, float eps) {
    constexpr int PER = DV / 64;  // elements per lane
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t off = row * DV + lane * PER;
    const Vec<OT, PER> ov = load_vec<OT, PER>(o + off);
    const Vec<In, PER> zv = load_vec<In, PER>(z + off);
    float x[PER], s = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        x[e] = to_f32(ov.v[e]);
        s += x[e] * x[e];
    }
    s = wave_sum(s);
    const float inv = 1.f / sqrtf(s * (1.f / DV) + eps);
    float r[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) r[e] = x[e] * inv * gamma[lane * PER + e] * silu_f(to_f32(zv.v[e]));
    if constexpr (PER == 1) {
        y[off] = from_f32<In>(r[0]);
    } else {
        typedef In V __attribute__((ext_vector_type(PER)));
        V out;
#pragma unroll
        for (int e = 0; e < PER; ++e) out[e] = from_f32<In>(r[e]);
        *reinterpret_cast<V*>(y + off) = out;
    }
}

template <typename In, int D>
hipError_t launch_prep_t(const MixerPrepArgs& a) {
    const int nblk = (int)((a.T + TBK - 1) / TBK);
    hipLaunchKernelGGL((prep_kernel<In, D, D>), dim3((unsigned)(a.B * a.H * nblk)), dim3(2 * D), 0,
                       (hipStream_t)a.stream, (const In*)a.xq, (const In*)a.xk, (const In*)a.xv, (const In*)a.xb,
                       (const In*)a.xw, (const In*)a.xa, a.conv_q, a.conv_k, a.conv_v, (In*)a.q, (In*)a.k, (In*)a.v,
                       (In*)a.b, (In*)a.w, a.log_alpha, (int)a.T, (int)a.H, nblk, a.eps);
    return hipGetLastError();
}

template <typename OT, typename In, int D>
hipError_t launch_out_t(const MixerOutArgs& a) {
    const int64_t rows = a.B * a.T * a.H;
    hipLaunchKernelGGL((out_kernel<OT, In, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       (hipStream_t)a.stream, (const OT*)a.o, (const In*)a.z, a.gamma, (In*)a.y, rows, a.eps);
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
