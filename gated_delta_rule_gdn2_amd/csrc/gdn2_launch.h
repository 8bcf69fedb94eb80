// gdn2_launch.h -- host-side launch entry points of the kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const void* b;
    const void* w;
    const float* initial_state;
    void* o;
    float* final_state;
    int64_t B, T, H, dk, dv;
    bool dtype_bf16;  // inputs q, k, v, b, w are bf16 (else fp32)
    bool out_f32;     // o is fp32 (else the input dtype)
    void* stream;
    // packed sequences: B + 1 offsets into the token axis of length T (device memory), or
    // nullptr for B sequences of T tokens each
    const int64_t* cu_seqlens = nullptr;
    int cus = 256;  // compute units of the device
    // gate logits instead of activated gates (bf16 inputs only): decay_logits [.., dk] holds a
    // with alpha = sigmoid(a), and b, w hold logits xb, xw with b = sigmoid(xb), w = sigmoid(xw);
    // log_alpha is then unused
    bool gate_logits = false;
    const void* decay_logits = nullptr;
    const void* decay() const { return gate_logits ? decay_logits : (const void*)log_alpha; }
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const void* b;
    const void* w;
    float* state;
    void* o;
    int64_t N, H, dk, dv;
    bool dtype_bf16;
    bool out_f32;
    void* stream;
};

// Floats of the backward's per-chunk record (64-token chunks): T and P (64 x 64), W and KR
// (64 x dk, row-major and swizzled), QG (64 x dk, swizzled), U0 (64 x dv), Gamma_C (dk),
// rounded up to 256 bytes.
constexpr int64_t bwd_rec_floats(int64_t dk, int64_t dv) {
    return (2 * 64 * 64 + 5 * 64 * dk + 64 * dv + dk + 63) / 64 * 64;
}

// Backward pass (vector-Jacobian product) of the chunk forward, fixed-length sequences.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const void* b;
    const void* w;
    const float* initial_state;  // or nullptr (zeros)
    const float* d_o;            // [B,T,H,dv] fp32
    const float* d_final_state;  // [B,H,dk,dv] fp32 or nullptr (zeros)
    // gradients, fp32, laid out like their inputs; g_s0 may be nullptr
    float* g_q;
    float* g_k;
    float* g_v;
    float* g_log_alpha;
    float* g_b;
    float* g_w;
    float* g_s0;
    // workspace (fp32): states entering every chunk and dS' of every chunk [B,H,NC,dk,dv],
    // U and dR [B,T,H,dv], one record of chunk-local quantities per chunk [B,H,NC,
    // bwd_rec_floats(dk, dv)]
    float* s_ckpt;
    float* ds_ckpt;
    float* u;
    float* dr;
    float* loc;
    int64_t B, T, H, dk, dv;
    bool dtype_bf16;
    void* stream;
    int cus;  // compute units of the device
};

// The mixer's fused elementwise passes before and after the recurrence.
struct MixerPrepArgs {
    const void* xq;
    const void* xk;
    const void* xv;
    const void* xb;
    const void* xw;
    const void* xa;
    const float* conv_q;  // [H*dk][4]
    const float* conv_k;  // [H*dk][4]
    const float* conv_v;  // [H*dv][4]
    void* q;
    void* k;
    void* v;
    void* b;
    void* w;
    float* log_alpha;
    int64_t B, T, H, dk, dv;
    bool dtype_bf16;
    float eps;
    void* stream;
};

struct MixerOutArgs {
    const void* o;
    const void* z;
    const float* gamma;  // [dv]
    void* y;
    int64_t B, T, H, dv;
    bool dtype_bf16;  // z and y (and o unless o_f32)
    bool o_f32;
    float eps;
    void* stream;
};

// dvs: value columns per workgroup slice (16, 32 or 64)
hipError_t launch_chunk_fwd(const ChunkArgs& a, int dvs);
// The forward in two kernels (chunk-local records, then the state pass), bf16 inputs with
// dk = dv = 64 or 128, fixed-length sequences; workspace of split_workspace_bytes bytes (which
// depends on the compute units: with few chains the form cuts sequences into segments).
size_t split_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d, int64_t cus);
hipError_t launch_chunk_split(const ChunkArgs& a, void* workspace);
// bf16 inputs (dk = dv = 64 or 128)
hipError_t launch_chunk_bf16(const ChunkArgs& a, int dvs);
hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_chunk_bwd(const BwdArgs& a);
hipError_t launch_mixer_prep(const MixerPrepArgs& a);
hipError_t launch_mixer_out(const MixerOutArgs& a);

}  // namespace gdn2
