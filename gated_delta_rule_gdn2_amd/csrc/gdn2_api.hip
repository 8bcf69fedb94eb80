// gdn2_api.hip -- the exported C ABI (include/gdn2.h): argument validation,
// choice of the launch configuration, and dispatch to the kernels.
//
// Everything here runs on the host.  Validation is complete before any HIP
// call, so an invalid call enqueues nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <mutex>

#include "../../include/gdn2.h"
#include "gdn2_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool chunk_supported(int64_t dk, int64_t dv, gdn2_dtype_t dt) {
    if (dt == GDN2_DTYPE_BF16) return (dk == 128 && dv == 128) || (dk == 64 && dv == 64);
    if (dt == GDN2_DTYPE_F32) return dk == 64 && dv == 64;
    return false;
}
// the two-kernel forward: bf16 inputs, dk = dv = 64 or 128, sequences of one length
bool split_supported(bool packed, int64_t dk, int64_t dv, gdn2_dtype_t dt) {
    return !packed && dt == GDN2_DTYPE_BF16 && dk == dv && (dk == 64 || dk == 128);
}
bool mixer_supported(int64_t dk, int64_t dv, gdn2_dtype_t dt) {
    if (dt != GDN2_DTYPE_BF16 && dt != GDN2_DTYPE_F32) return false;
    return (dk == 128 && dv == 128) || (dk == 64 && dv == 64);
}
bool decode_supported(int64_t dk, int64_t dv, gdn2_dtype_t dt) {
    if (dt != GDN2_DTYPE_BF16 && dt != GDN2_DTYPE_F32) return false;
    return (dk == 128 && dv == 128) || (dk == 64 && dv == 64);
}

// Value columns per workgroup.  The columns of the state evolve independently,
// so a (sequence, head) splits into dv / dvs workgroups; the smallest power of
// two of slices that gives at least one workgroup per compute unit is taken
// (more slices repeat the key-side work of every chunk in every slice).  A
// slice holds at most 64 columns (LDS budget).
int choose_dvs(int64_t BH, int64_t dv, int cus) {
    const int64_t max_slices = dv / 16;
    const int64_t min_slices = dv / 64;
    int64_t s = min_slices < 1 ? 1 : min_slices;
    while (s < max_slices && BH * s < cus) s *= 2;
    return static_cast<int>(dv / s);
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    return cus;
}

// Workspace of the backward pass: byte offsets of its five fp32 parts, each rounded up to 256
// bytes.  False if the sizes overflow (or a head dimension exceeds 2^20).
struct BwdLayout {
    int64_t s_ckpt, ds_ckpt, u, dr, loc, total;
};
bool bwd_layout(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, BwdLayout* l) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0 || dk > (1 << 20) || dv > (1 << 20)) return false;
    const int64_t nc = (T + 63) / 64;
    int64_t bh, bhn, st, btv, tpn;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, nc, &bhn) || !mul_ok(bhn, dk * dv, &st) || !mul_ok(st, 4, &st))
        return false;
    if (!mul_ok(B * H, T, &btv) || !mul_ok(btv, dv * 4, &btv)) return false;
    if (!mul_ok(bhn, gdn2::bwd_rec_floats(dk, dv) * 4, &tpn)) return false;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    if (st > INT64_MAX / 8 || btv > INT64_MAX / 8 || tpn > INT64_MAX / 8) return false;
    l->s_ckpt = 0;
    l->ds_ckpt = up(st);
    l->u = l->ds_ckpt + up(st);
    l->dr = l->u + up(btv);
    l->loc = l->dr + up(btv);
    l->total = l->loc + up(tpn);
    return true;
}

// Validation and launch shared by the fixed-length and the packed-sequence forward.  NS
// sequences (states [NS, H, dk, dv]); the token tensors hold NT tokens in all; T_or_total is
// the kernels' token parameter (T per sequence, or the packed total).  decay is log alpha
// (fp32), or with logits the decay logits in the input dtype, and b, w are then gate logits.
gdn2_status_t chunk_fwd_common(const void* q, const void* k, const void* v, const void* decay,
                               const void* b, const void* w, const float* initial_state, void* o,
                               float* final_state, const int64_t* cu_seqlens, int64_t NS,
                               int64_t T_or_total, int64_t NT, int64_t H, int64_t dk, int64_t dv,
                               gdn2_dtype_t dtype, gdn2_dtype_t o_dtype, void* workspace,
                               size_t workspace_bytes, void* stream, bool logits = false) {
    if (!q || !k || !v || !decay || !b || !w || !o) return GDN2_ERR_NULL;
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_UNSUPPORTED;
    if (logits && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_UNSUPPORTED;
    if (o_dtype != GDN2_DTYPE_F32 && o_dtype != dtype) return GDN2_ERR_UNSUPPORTED;
    if (H < 1 || dk < 1 || dv < 1) return GDN2_ERR_SHAPE;
    if (!chunk_supported(dk, dv, dtype)) return GDN2_ERR_UNSUPPORTED;
    // sizes: kernels index rows with 32-bit sequence, token and head counts and 64-bit
    // element offsets
    int64_t NTH, nk, nv, ns;
    if (NS > INT_MAX || T_or_total > INT_MAX || H > INT_MAX) return GDN2_ERR_SHAPE;
    if (!mul_ok(NT, H, &NTH) || !mul_ok(NTH, dk, &nk) || !mul_ok(NTH, dv, &nv)) return GDN2_ERR_SHAPE;
    if (!mul_ok(NS * H, dk * dv, &ns)) return GDN2_ERR_SHAPE;
    if (NS * H * (dv / 16) > UINT_MAX / 2) return GDN2_ERR_SHAPE;
    // per-lane offsets inside one chunk are formed with 24-bit multiplies of the token stride
    // per-lane 32-bit byte offsets within a chunk (64 tokens of up to 4-byte elements) and the
    // chunk's buffer range stay below 2^30
    if (H * dk >= (int64_t(1) << 22) || H * dv >= (int64_t(1) << 22)) return GDN2_ERR_SHAPE;
    const void* ptrs[] = {q, k, v, decay, b, w, initial_state, o, final_state};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    const int64_t es = dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const int64_t eo = o_dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const Range in_ranges[] = {range_of(q, nk * es), range_of(k, nk * es), range_of(v, nv * es),
                               range_of(decay, nk * (logits ? es : 4)), range_of(b, nk * es),
                               range_of(w, nv * es)};
    const Range ro = range_of(o, nv * eo);
    for (const Range& r : in_ranges)
        if (overlap(ro, r)) return GDN2_ERR_ALIAS;
    if (initial_state && overlap(ro, range_of(initial_state, ns * 4))) return GDN2_ERR_ALIAS;
    const Range rc = range_of(cu_seqlens, cu_seqlens ? (NS + 1) * 8 : 0);
    if (overlap(ro, rc)) return GDN2_ERR_ALIAS;
    if (final_state) {
        const Range rf = range_of(final_state, ns * 4);
        for (const Range& r : in_ranges)
            if (overlap(rf, r)) return GDN2_ERR_ALIAS;
        if (overlap(rf, ro) || overlap(rf, rc)) return GDN2_ERR_ALIAS;
        if (initial_state && initial_state != final_state && overlap(rf, range_of(initial_state, ns * 4)))
            return GDN2_ERR_ALIAS;
    }
    // the two-kernel path when the caller passes its workspace, else the single fused kernel
    const bool split = workspace != nullptr || workspace_bytes != 0;
    if (split) {
        const size_t need = split_supported(cu_seqlens != nullptr, dk, dv, dtype)
                                ? gdn2_chunk_fwd_split_workspace_bytes(NS, T_or_total, H, dk, dv, dtype) : 0;
        if (need == 0) return GDN2_ERR_WORKSPACE;  // this call takes no workspace
        if (!workspace || workspace_bytes < need) return GDN2_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) & 255u) return GDN2_ERR_MISALIGNED;
        const Range rw = range_of(workspace, (int64_t)need);
        for (const Range& r : in_ranges)
            if (overlap(rw, r)) return GDN2_ERR_ALIAS;
        if (overlap(rw, ro) || (initial_state && overlap(rw, range_of(initial_state, ns * 4))) ||
            (final_state && overlap(rw, range_of(final_state, ns * 4))))
            return GDN2_ERR_ALIAS;
    }
    if (NT == 0 && !final_state) return GDN2_OK;  // nothing to compute or write
    const int cus = device_cus();
    if (cus <= 0) return GDN2_ERR_HIP;
    gdn2::ChunkArgs a{q, k, v, logits ? nullptr : static_cast<const float*>(decay), b, w, initial_state, o,
                      final_state, NS, T_or_total, H, dk, dv, dtype == GDN2_DTYPE_BF16,
                      o_dtype == GDN2_DTYPE_F32, stream, cu_seqlens, cus};
    a.gate_logits = logits;
    a.decay_logits = logits ? decay : nullptr;
    if (split) return gdn2::launch_chunk_split(a, workspace) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
    const int dvs = choose_dvs(NS * H, dv, cus);
    return gdn2::launch_chunk_fwd(a, dvs) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

// The allocation-free backward: its workspace is this file-scope device array, one per GPU the
// library runs on (held until the process ends).  Host code never uses the array's name as an
// address: each device's address is looked up once, with that device current, and kept.
constexpr size_t kScratchBytes = GDN2_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of the scratch array (looked up on the first call on the device).
gdn2_status_t scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN2_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN2_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return GDN2_OK;
}

gdn2_status_t chunk_bwd_common(const void* q, const void* k, const void* v, const float* log_alpha,
                             const void* b, const void* w, const float* initial_state, const float* d_o,
                             const float* d_final_state, float* dq, float* dk, float* dv, float* dlog_alpha,
                             float* db, float* dw, float* d_initial_state, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t T, int64_t H, int64_t dk_dim,
                             int64_t dv_dim, gdn2_dtype_t dtype, void* stream, bool use_scratch) {
    if (!q || !k || !v || !log_alpha || !b || !w || !d_o) return GDN2_ERR_NULL;
    if (!dq || !dk || !dv || !dlog_alpha || !db || !dw) return GDN2_ERR_NULL;
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || dk_dim < 1 || dv_dim < 1) return GDN2_ERR_SHAPE;
    if (!chunk_supported(dk_dim, dv_dim, dtype)) return GDN2_ERR_UNSUPPORTED;
    int64_t BT, NTH, nk, nv, ns;
    if (B > INT_MAX || T > INT_MAX || H > INT_MAX) return GDN2_ERR_SHAPE;
    if (!mul_ok(B, T, &BT) || !mul_ok(BT, H, &NTH) || !mul_ok(NTH, dk_dim, &nk) || !mul_ok(NTH, dv_dim, &nv))
        return GDN2_ERR_SHAPE;
    if (!mul_ok(B * H, dk_dim * dv_dim, &ns)) return GDN2_ERR_SHAPE;
    if (H * dk_dim >= (int64_t(1) << 24) || H * dv_dim >= (int64_t(1) << 24)) return GDN2_ERR_SHAPE;
    BwdLayout l;
    if (!bwd_layout(B, T, H, dk_dim, dv_dim, &l)) return GDN2_ERR_SHAPE;
    if (B * H * ((T + 63) / 64) > UINT_MAX / 2 || B * H * (dv_dim / 16) > UINT_MAX / 2) return GDN2_ERR_SHAPE;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv,
                          dlog_alpha, db, dw, d_initial_state};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    if (use_scratch) {
        // the scratch array is a separate allocation, so it overlaps no argument
        if ((size_t)l.total > kScratchBytes) return GDN2_ERR_WORKSPACE;
        const gdn2_status_t st = scratch_address(&workspace);
        if (st != GDN2_OK) return st;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < (size_t)l.total) return GDN2_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GDN2_ERR_MISALIGNED;
    const int64_t es = dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const Range ins[] = {range_of(q, nk * es), range_of(k, nk * es), range_of(v, nv * es),
                         range_of(log_alpha, nk * 4), range_of(b, nk * es), range_of(w, nv * es),
                         range_of(initial_state, initial_state ? ns * 4 : 0), range_of(d_o, nv * 4),
                         range_of(d_final_state, d_final_state ? ns * 4 : 0)};
    const Range outs[] = {range_of(dq, nk * 4), range_of(dk, nk * 4), range_of(dv, nv * 4),
                          range_of(dlog_alpha, nk * 4), range_of(db, nk * 4), range_of(dw, nv * 4),
                          range_of(d_initial_state, d_initial_state ? ns * 4 : 0), range_of(workspace, l.total)};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return GDN2_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(outs[i], outs[j])) return GDN2_ERR_ALIAS;
    }
    const int cus = device_cus();
    if (cus <= 0) return GDN2_ERR_HIP;
    char* ws = static_cast<char*>(workspace);
    gdn2::BwdArgs a{q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv, dlog_alpha, db,
                    dw, d_initial_state, reinterpret_cast<float*>(ws + l.s_ckpt),
                    reinterpret_cast<float*>(ws + l.ds_ckpt), reinterpret_cast<float*>(ws + l.u),
                    reinterpret_cast<float*>(ws + l.dr), reinterpret_cast<float*>(ws + l.loc), B, T, H, dk_dim,
                    dv_dim, dtype == GDN2_DTYPE_BF16, stream, cus};
    return gdn2::launch_chunk_bwd(a) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

}  // namespace

extern "C" {

size_t gdn2_chunk_fwd_split_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                            gdn2_dtype_t dtype) {
    if (!split_supported(false, dk, dv, dtype) || B < 1 || T < 1 || H < 1 || B > INT_MAX || T > INT_MAX ||
        H > INT_MAX || B * H > INT_MAX / 64)
        return 0;
    const int cus = device_cus();
    return gdn2::split_workspace_bytes(B, T, H, dk, cus > 0 ? cus : 256);
}

size_t gdn2_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      gdn2_dtype_t dtype) {
    // The fused kernel walks each (sequence, head, 64-column slice) on one compute unit; when
    // those chains cannot fill the GPU, the two-kernel form is faster (its chunk-local work is
    // spread over every chunk).  Below that point the fused kernel needs no workspace.
    const int64_t cus = device_cus() > 0 ? device_cus() : 256;
    if (B < 1 || H < 1 || B > INT_MAX || H > INT_MAX || B * H * ((dv + 63) / 64) >= cus) return 0;
    return gdn2_chunk_fwd_split_workspace_bytes(B, T, H, dk, dv, dtype);
}

gdn2_status_t gdn2_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                             const void* b, const void* w, const float* initial_state, void* o,
                             float* final_state, int64_t B, int64_t T, int64_t H, int64_t dk,
                             int64_t dv, gdn2_dtype_t dtype, gdn2_dtype_t o_dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (B < 1 || T < 1) return GDN2_ERR_SHAPE;
    int64_t BT;
    if (!mul_ok(B, T, &BT)) return GDN2_ERR_SHAPE;
    return chunk_fwd_common(q, k, v, log_alpha, b, w, initial_state, o, final_state, nullptr, B, T, BT, H,
                            dk, dv, dtype, o_dtype, workspace, workspace_bytes, stream);
}

gdn2_status_t gdn2_chunk_fwd_logits(const void* q, const void* k, const void* v, const void* a_logit,
                                    const void* b_logit, const void* w_logit, const float* initial_state,
                                    void* o, float* final_state, int64_t B, int64_t T, int64_t H, int64_t dk,
                                    int64_t dv, gdn2_dtype_t dtype, gdn2_dtype_t o_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (B < 1 || T < 1) return GDN2_ERR_SHAPE;
    int64_t BT;
    if (!mul_ok(B, T, &BT)) return GDN2_ERR_SHAPE;
    return chunk_fwd_common(q, k, v, a_logit, b_logit, w_logit, initial_state, o, final_state, nullptr, B, T,
                            BT, H, dk, dv, dtype, o_dtype, workspace, workspace_bytes, stream, true);
}

gdn2_status_t gdn2_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                                    const void* b, const void* w, const float* initial_state, void* o,
                                    float* final_state, const int64_t* cu_seqlens, int64_t N,
                                    int64_t total_T, int64_t H, int64_t dk, int64_t dv,
                                    gdn2_dtype_t dtype, gdn2_dtype_t o_dtype, void* stream) {
    if (!cu_seqlens) return GDN2_ERR_NULL;
    if (N < 1 || total_T < 0) return GDN2_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) return GDN2_ERR_MISALIGNED;
    return chunk_fwd_common(q, k, v, log_alpha, b, w, initial_state, o, final_state, cu_seqlens, N, total_T,
                            total_T, H, dk, dv, dtype, o_dtype, nullptr, 0, stream);
}

gdn2_status_t gdn2_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                               const void* b, const void* w, float* state, void* o, int64_t N,
                               int64_t H, int64_t dk, int64_t dv, gdn2_dtype_t dtype,
                               gdn2_dtype_t o_dtype, void* stream) {
    if (!q || !k || !v || !log_alpha || !b || !w || !state || !o) return GDN2_ERR_NULL;
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_UNSUPPORTED;
    if (o_dtype != GDN2_DTYPE_F32 && o_dtype != dtype) return GDN2_ERR_UNSUPPORTED;
    if (N < 1 || H < 1 || dk < 1 || dv < 1) return GDN2_ERR_SHAPE;
    if (!decode_supported(dk, dv, dtype)) return GDN2_ERR_UNSUPPORTED;
    int64_t NH, nk, nv, ns;
    if (!mul_ok(N, H, &NH) || !mul_ok(NH, dk, &nk) || !mul_ok(NH, dv, &nv) || !mul_ok(NH, dk * dv, &ns))
        return GDN2_ERR_SHAPE;
    if (NH > UINT_MAX / 2) return GDN2_ERR_SHAPE;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, state, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN2_ERR_MISALIGNED;
    const int64_t es = dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const Range in_ranges[] = {range_of(q, nk * es), range_of(k, nk * es), range_of(v, nv * es),
                               range_of(log_alpha, nk * 4), range_of(b, nk * es),
                               range_of(w, nv * es)};
    const int64_t eo = o_dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const Range ro = range_of(o, nv * eo), rs = range_of(state, ns * 4);
    for (const Range& r : in_ranges)
        if (overlap(ro, r) || overlap(rs, r)) return GDN2_ERR_ALIAS;
    if (overlap(ro, rs)) return GDN2_ERR_ALIAS;
    gdn2::DecodeArgs a{q, k, v, log_alpha, b, w, state, o, N, H, dk, dv, dtype == GDN2_DTYPE_BF16,
                       o_dtype == GDN2_DTYPE_F32, stream};
    return gdn2::launch_decode_step(a) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

size_t gdn2_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
    BwdLayout l;
    return bwd_layout(B, T, H, dk, dv, &l) ? (size_t)l.total : 0;
}

gdn2_status_t gdn2_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
                             const void* b, const void* w, const float* initial_state, const float* d_o,
                             const float* d_final_state, float* dq, float* dk, float* dv, float* dlog_alpha,
                             float* db, float* dw, float* d_initial_state, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t T, int64_t H, int64_t dk_dim,
                             int64_t dv_dim, gdn2_dtype_t dtype, void* stream) {
    return chunk_bwd_common(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv, dlog_alpha,
                            db, dw, d_initial_state, workspace, workspace_bytes, B, T, H, dk_dim, dv_dim, dtype,
                            stream, false);
}

gdn2_status_t gdn2_chunk_bwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                     const void* b, const void* w, const float* initial_state,
                                     const float* d_o, const float* d_final_state, float* dq, float* dk,
                                     float* dv, float* dlog_alpha, float* db, float* dw,
                                     float* d_initial_state, int64_t B, int64_t T, int64_t H,
                                     int64_t dk_dim, int64_t dv_dim, gdn2_dtype_t dtype, void* stream) {
    return chunk_bwd_common(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv, dlog_alpha,
                            db, dw, d_initial_state, nullptr, 0, B, T, H, dk_dim, dv_dim, dtype, stream, true);
}

gdn2_status_t gdn2_mixer_prep(const void* xq, const void* xk, const void* xv, const void* xb, const void* xw,
                              const void* xa, const float* conv_q, const float* conv_k, const float* conv_v,
                              void* q, void* k, void* v, void* b, void* w, float* log_alpha, int64_t B,
                              int64_t T, int64_t H, int64_t dk, int64_t dv, float eps, gdn2_dtype_t dtype,
                              void* stream) {
    // b, w and log_alpha all NULL: the gates are left to gdn2_chunk_fwd_logits (xb, xw, xa unused)
    const bool gates = b || w || log_alpha;
    if (!gates) xb = xw = xa = nullptr;
    if (!xq || !xk || !xv || !conv_q || !conv_k || !conv_v || !q || !k || !v) return GDN2_ERR_NULL;
    if (gates && (!xb || !xw || !xa || !b || !w || !log_alpha)) return GDN2_ERR_NULL;
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1 || !(eps >= 0.f) || eps > 1e30f) return GDN2_ERR_SHAPE;
    if (!mixer_supported(dk, dv, dtype)) return GDN2_ERR_UNSUPPORTED;
    int64_t BT, nk, nv, blocks;
    if (B > INT_MAX || T > INT_MAX || H > INT_MAX) return GDN2_ERR_SHAPE;
    if (!mul_ok(B, T, &BT) || !mul_ok(BT, H * dk, &nk) || !mul_ok(BT, H * dv, &nv)) return GDN2_ERR_SHAPE;
    // workgroups: B x ceil(T / 4) x ceil(H / heads per wave), bounded here by B H ceil(T / 4)
    if (!mul_ok(B * H, (T + 3) / 4, &blocks) || blocks > INT_MAX) return GDN2_ERR_SHAPE;
    const void* ptrs[] = {xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, q, k, v, b, w, log_alpha};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN2_ERR_MISALIGNED;
    const int64_t es = dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const int64_t gk = gates ? nk : 0, gv = gates ? nv : 0;  // gate tensors: empty ranges when absent
    const Range ins[] = {range_of(xq, nk * es), range_of(xk, nk * es), range_of(xv, nv * es), range_of(xb, gk * es),
                         range_of(xw, gv * es), range_of(xa, gk * es), range_of(conv_q, H * dk * 16),
                         range_of(conv_k, H * dk * 16), range_of(conv_v, H * dv * 16)};
    const Range outs[] = {range_of(q, nk * es), range_of(k, nk * es), range_of(v, nv * es), range_of(b, gk * es),
                          range_of(w, gv * es), range_of(log_alpha, gk * 4)};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return GDN2_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(outs[i], outs[j])) return GDN2_ERR_ALIAS;
    }
    gdn2::MixerPrepArgs a{xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, q, k, v, b, w, log_alpha,
                          B, T, H, dk, dv, dtype == GDN2_DTYPE_BF16, eps, stream};
    return gdn2::launch_mixer_prep(a) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status_t gdn2_mixer_out(const void* o, const void* z, const float* gamma, void* y, int64_t B, int64_t T,
                             int64_t H, int64_t dv, float eps, gdn2_dtype_t dtype, gdn2_dtype_t o_dtype,
                             void* stream) {
    if (!o || !z || !gamma || !y) return GDN2_ERR_NULL;
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_UNSUPPORTED;
    if (o_dtype != GDN2_DTYPE_F32 && o_dtype != dtype) return GDN2_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || dv < 1 || !(eps >= 0.f) || eps > 1e30f) return GDN2_ERR_SHAPE;
    if (!mixer_supported(dv, dv, dtype)) return GDN2_ERR_UNSUPPORTED;
    int64_t rows, nv;
    if (!mul_ok(B, T, &rows) || !mul_ok(rows, H, &rows) || !mul_ok(rows, dv, &nv)) return GDN2_ERR_SHAPE;
    if ((rows + 3) / 4 > INT_MAX) return GDN2_ERR_SHAPE;
    const void* ptrs[] = {o, z, gamma, y};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN2_ERR_MISALIGNED;
    const int64_t es = dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const int64_t eo = o_dtype == GDN2_DTYPE_BF16 ? 2 : 4;
    const Range ry = range_of(y, nv * es);
    if (overlap(ry, range_of(o, nv * eo)) || overlap(ry, range_of(z, nv * es)) || overlap(ry, range_of(gamma, dv * 4)))
        return GDN2_ERR_ALIAS;
    gdn2::MixerOutArgs a{o, z, gamma, y, B, T, H, dv, dtype == GDN2_DTYPE_BF16, o_dtype == GDN2_DTYPE_F32, eps, stream};
    return gdn2::launch_mixer_out(a) == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_supported(int which, int64_t dk, int64_t dv, gdn2_dtype_t dtype) {
    if (which == 3) return mixer_supported(dk, dv, dtype) ? 1 : 0;
    if (which == 0 || which == 2) return chunk_supported(dk, dv, dtype) ? 1 : 0;
    if (which == 1) return decode_supported(dk, dv, dtype) ? 1 : 0;
    return 0;
}

const char* gdn2_status_string(gdn2_status_t s) {
    switch (s) {
        case GDN2_OK: return "ok";
        case GDN2_ERR_NULL: return "a required pointer is NULL";
        case GDN2_ERR_SHAPE: return "a size is out of range";
        case GDN2_ERR_UNSUPPORTED: return "(dk, dv, dtype) is not supported";
        case GDN2_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
        case GDN2_ERR_ALIAS: return "an output overlaps an input";
        case GDN2_ERR_WORKSPACE: return "the workspace is missing or too small";
        case GDN2_ERR_HIP: return "the HIP runtime rejected the call";
    }
    return "unknown status";
}

const char* gdn2_version(void) { return "gdn2-gfx950 0.1.0"; }

}  // extern "C"
