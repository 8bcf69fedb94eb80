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
    // U and dR [B,T,H,dv], T and P of every chunk [B,H,NC,2,64,64]
    float* s_ckpt;
    float* ds_ckpt;
    float* u;
    float* dr;
    float* tp;
    int64_t B, T, H, dk, dv;
    bool dtype_bf16;
    void* stream;
    int cus;  // compute units of the device
};

// dvs: value columns per workgroup slice (16, 32 or 64)
hipError_t launch_chunk_fwd(const ChunkArgs& a, int dvs);
// bf16 inputs (dk = dv = 64 or 128)
hipError_t launch_chunk_bf16(const ChunkArgs& a, int dvs);
hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_chunk_bwd(const BwdArgs& a);

}  // namespace gdn2
