// gdn2_decode.hip -- single-token recurrent step of GDN-2 on gfx950.
//
// One step of the recurrence of the page "Why NVIDIA Gated DeltaNet-2
// separates erase and write gates" (axbrief.com), section "Gated Delta
// Rule-2", in the residual form the same section describes (decayed state,
// gated read, gated residual written along k), with a constant-size state:
//
//   S' = Diag(alpha) S;  r = S'^T (b.k);  s = S'^T q;  u = w.v - r;
//   S  <- S' + k u^T;    o = S^T q = s + (k.q) u.
//
// The step reads and writes each state element exactly once, so it is bound
// by HBM bandwidth: 2 * dk * dv * 4 bytes of state per (sequence, head) plus
// the token vectors.  One workgroup of 256 threads owns one (n, h) state; a
// thread holds a float4 column quad on dk*dv/1024 rows in registers, the two
// column reductions over dk go through LDS, and the update is written back in
// place.
#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {

template <typename T, typename OutT, int DK, int DV>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const T* __restrict__ bgate, const T* __restrict__ wgate,
    float* __restrict__ state, OutT* __restrict__ o) {
    constexpr int NQ = DV / 4;        // float4 column quads per row
    constexpr int NRG = 256 / NQ;     // row groups
    constexpr int RPG = DK / NRG;     // rows per thread
    static_assert(RPG * NRG == DK && NQ * NRG == 256, "decode tiling");
    __shared__ float s_alpha[DK], s_bk[DK], s_q[DK], s_k[DK];
    __shared__ __attribute__((aligned(16))) float s_red[NRG][2 * DV];
    __shared__ float s_kq[NRG];

    const int tid = threadIdx.x;
    const int64_t nh = blockIdx.x;  // n * H + h
    const int cq = tid % NQ;
    const int rg = tid / NQ;

    // token vectors (key side) into LDS
    for (int c = tid; c < DK; c += 256) {
        const int64_t off = nh * DK + c;
        const float kk = to_f32(k[off]);
        s_alpha[c] = exp_neg(log_alpha[off]);
        s_bk[c] = to_f32(bgate[off]) * kk;
        s_q[c] = to_f32(q[off]);
        s_k[c] = kk;
    }
    // this thread's rows of the state
    float4 sv[RPG];
    float* base = state + nh * DK * DV + (int64_t)(rg * RPG) * DV + cq * 4;
#pragma unroll
    for (int i = 0; i < RPG; ++i) sv[i] = *reinterpret_cast<const float4*>(base + (int64_t)i * DV);
    __syncthreads();

    // decay rows, partial column reductions r = S'^T (b.k), s = S'^T q, and k.q
    float r4[4] = {0.f, 0.f, 0.f, 0.f}, s4[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
        const int row = rg * RPG + i;
        const float a = s_alpha[row], bkr = s_bk[row], qr = s_q[row];
        sv[i].x *= a; sv[i].y *= a; sv[i].z *= a; sv[i].w *= a;
        r4[0] += sv[i].x * bkr; r4[1] += sv[i].y * bkr; r4[2] += sv[i].z * bkr; r4[3] += sv[i].w * bkr;
        s4[0] += sv[i].x * qr; s4[1] += sv[i].y * qr; s4[2] += sv[i].z * qr; s4[3] += sv[i].w * qr;
        kq += s_k[row] * qr;
    }
    *reinterpret_cast<float4*>(&s_red[rg][cq * 4]) = make_float4(r4[0], r4[1], r4[2], r4[3]);
    *reinterpret_cast<float4*>(&s_red[rg][DV + cq * 4]) = make_float4(s4[0], s4[1], s4[2], s4[3]);
    if (cq == 0) s_kq[rg] = kq;
    __syncthreads();

    float rt[4] = {0.f, 0.f, 0.f, 0.f}, st[4] = {0.f, 0.f, 0.f, 0.f}, kqt = 0.f;
#pragma unroll
    for (int gq = 0; gq < NRG; ++gq) {
        const float4 a = *reinterpret_cast<const float4*>(&s_red[gq][cq * 4]);
        const float4 b = *reinterpret_cast<const float4*>(&s_red[gq][DV + cq * 4]);
        rt[0] += a.x; rt[1] += a.y; rt[2] += a.z; rt[3] += a.w;
        st[0] += b.x; st[1] += b.y; st[2] += b.z; st[3] += b.w;
        kqt += s_kq[gq];
    }
    // gated residual for this thread's four columns
    float u[4];
    {
        const int64_t off = nh * DV + cq * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = to_f32(wgate[off + e]) * to_f32(v[off + e]) - rt[e];
    }
    // write along k, in place
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
        const float kr = s_k[rg * RPG + i];
        float4 x = sv[i];
        x.x += kr * u[0]; x.y += kr * u[1]; x.z += kr * u[2]; x.w += kr * u[3];
        *reinterpret_cast<float4*>(base + (int64_t)i * DV) = x;
    }
    if (rg == 0) {
        const int64_t off = nh * DV + cq * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[off + e] = from_f32<OutT>(st[e] + kqt * u[e]);
    }
}

template <typename T, typename OutT, int DK, int DV>
static hipError_t launch_dec(const DecodeArgs& a) {
    const int64_t groups = a.N * a.H;
    hipLaunchKernelGGL((decode_step_kernel<T, OutT, DK, DV>), dim3((unsigned)groups), dim3(256), 0,
                       (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha,
                       (const T*)a.b, (const T*)a.w, a.state, (OutT*)a.o);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dec_d(const DecodeArgs& a) {
    if (!a.dtype_bf16) return launch_dec<float, float, D, D>(a);
    return a.out_f32 ? launch_dec<bf16, float, D, D>(a) : launch_dec<bf16, bf16, D, D>(a);
}

hipError_t launch_decode_step(const DecodeArgs& a) {
    if (a.dk == 128 && a.dv == 128) return launch_dec_d<128>(a);
    if (a.dk == 64 && a.dv == 64) return launch_dec_d<64>(a);
    return hipErrorInvalidValue;
}

}  // namespace gdn2
