// kda_api.cpp -- the extern "C" boundary of libkda.so: argument validation, dispatch, status.
// Declarations, layouts and error behaviour are documented in include/kda.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.hpp"

namespace {

constexpr int kVersion = 220;  // 0.2.2

bool valid_dtype(int dt) { return dt == KDA_F32 || dt == KDA_BF16; }
int64_t esize(int dt) { return dt == KDA_F32 ? 4 : 2; }
bool supported_d(int32_t d) { return d == 64 || d == 128; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes > 0 ? bytes : 0)};
}
bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// ---- the prefill workspace of kda_chunk_fwd_gated_noalloc: a static device array ------------
// Each GPU the library runs on holds its own copy from the first use on that device until the
// process ends.  In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to kernels.
__device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to.
hipError_t scratch_address(hipStream_t stream, void** out) {
    int dev = 0, cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        default: return "KDA_UNKNOWN_STATUS";
    }
}

int kda_version(void) { return kVersion; }

int kda_gate(const float* A, const void* z, int z_dtype, void* g, int g_dtype, int64_t n_tokens,
             int32_t H, int32_t dk, float g_min, void* stream) {
    if (!valid_dtype(z_dtype) || !valid_dtype(g_dtype) || n_tokens < 0 || H < 1 || dk < 1)
        return KDA_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(g_min) || !(g_min >= -5.0f && g_min < 0.0f)) return KDA_ERR_UNSUPPORTED;
    if (n_tokens == 0) return KDA_OK;
    if (!A || !z || !g) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t n = n_tokens * H * dk;
    const Range rg = range(g, n * esize(g_dtype));
    if (overlap(rg, range(z, n * esize(z_dtype))) || overlap(rg, range(A, int64_t(H) * dk * 4)))
        return KDA_ERR_INVALID_ARGUMENT;
    return from_hip(kda::launch_gate(A, z, z_dtype, g, g_dtype, n_tokens, H, dk, g_min,
                                     static_cast<hipStream_t>(stream)));
}

size_t kda_chunk_fwd_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dk,
                                    int32_t dv, int32_t chunk, int in_dtype) {
    if (n_seqs < 1 || total_tokens < 0 || H < 1 || !supported_d(dk) || !supported_d(dv) ||
        chunk != 64 || !valid_dtype(in_dtype))
        return 0;
    return kda::chunk_workspace_bytes(n_seqs, total_tokens, H, dk, dv, in_dtype);
}

}  // extern "C"

namespace {

// Validation and dispatch shared by kda_chunk_fwd (g given) and kda_chunk_fwd_gated (A, z given:
// gate_A != nullptr, g = z, g_dtype = z's dtype).
int chunk_fwd_impl(const void* q, const void* k, const void* v, const void* beta, int in_dtype,
                   const void* g, int g_dtype, const float* gate_A, float g_min,
                   const float* initial_state, float* final_state, const int32_t* cu_seqlens,
                   void* o, int o_dtype, int32_t B, int64_t T, int32_t n_seqs, int32_t H,
                   int32_t dk, int32_t dv, int32_t chunk, float scale, void* workspace,
                   size_t workspace_bytes, void* stream, bool gated, float* ckpt = nullptr,
                   int32_t ckpt_every = 0, int64_t ckpt_slots = 0, bool single_stream = false) {
    if (!valid_dtype(in_dtype) || !valid_dtype(g_dtype) || !valid_dtype(o_dtype))
        return KDA_ERR_INVALID_ARGUMENT;
    if (B < 1 || T < 0 || n_seqs < 1 || H < 1 || dk < 1 || dv < 1 || !std::isfinite(scale))
        return KDA_ERR_INVALID_ARGUMENT;
    if (cu_seqlens ? (B != 1) : (n_seqs != B)) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_d(dk) || !supported_d(dv) || chunk != 64) return KDA_ERR_UNSUPPORTED;
    if (gated && (!std::isfinite(g_min) || !(g_min >= -5.0f && g_min < 0.0f)))
        return KDA_ERR_UNSUPPORTED;
    const int64_t ntok = int64_t(B) * T;
    if (ntok > 0 && (!q || !k || !v || !beta || !g || !o || (gated && !gate_A)))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t need = kda::chunk_workspace_bytes(n_seqs, ntok, H, dk, dv, in_dtype);
    if (workspace_bytes < need || (need > 0 && !workspace)) return KDA_ERR_WORKSPACE;

    const int64_t state_bytes = int64_t(n_seqs) * H * dk * dv * 4;
    const Range r_q = range(q, ntok * H * dk * esize(in_dtype));
    const Range r_k = range(k, ntok * H * dk * esize(in_dtype));
    const Range r_v = range(v, ntok * H * dv * esize(in_dtype));
    const Range r_b = range(beta, ntok * H * esize(in_dtype));
    const Range r_g = range(g, ntok * H * dk * esize(g_dtype));
    const Range r_a = range(gate_A, gated && ntok > 0 ? int64_t(H) * dk * 4 : 0);
    const Range r_o = range(o, ntok * H * dv * esize(o_dtype));
    const Range r_h0 = range(initial_state, initial_state ? state_bytes : 0);
    const Range r_hT = range(final_state, final_state ? state_bytes : 0);
    const Range r_cu = range(cu_seqlens, cu_seqlens ? int64_t(n_seqs + 1) * 4 : 0);
    const Range r_ws = range(workspace, int64_t(workspace_bytes));
    const Range r_ck = range(ckpt, ckpt ? ckpt_slots * H * dk * dv * 4 : 0);
    for (const Range& x : {r_q, r_k, r_v, r_b, r_g, r_a, r_h0, r_hT, r_cu, r_ws, r_ck})
        if (overlap(r_o, x)) return KDA_ERR_INVALID_ARGUMENT;
    for (const Range& x : {r_q, r_k, r_v, r_b, r_g, r_a, r_h0, r_hT, r_cu, r_ws})
        if (overlap(r_ck, x)) return KDA_ERR_INVALID_ARGUMENT;
    // the final state may be the initial state itself, but must not partly overlap it
    if (initial_state && final_state && initial_state != final_state && overlap(r_h0, r_hT))
        return KDA_ERR_INVALID_ARGUMENT;
    for (const Range& x : {r_q, r_k, r_v, r_b, r_g, r_a, r_cu, r_ws})
        if (overlap(r_hT, x)) return KDA_ERR_INVALID_ARGUMENT;
    for (const Range& x : {r_q, r_k, r_v, r_b, r_g, r_a, r_h0, r_cu})
        if (overlap(r_ws, x)) return KDA_ERR_INVALID_ARGUMENT;

    if (kda::debug_validation_enabled() && ntok > 0) {
        bool ok = true;
        const hipError_t e = kda::debug_validate(gated ? nullptr : g, g_dtype, ntok * H * dk, cu_seqlens,
                                                 n_seqs, ntok, static_cast<hipStream_t>(stream), &ok);
        if (e != hipSuccess) return KDA_ERR_HIP;
        if (!ok) return KDA_ERR_INVALID_ARGUMENT;
    }

    kda::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g;
    a.gate_A = gated ? gate_A : nullptr; a.g_min = g_min;
    a.h0 = initial_state; a.hT = final_state; a.cu = cu_seqlens; a.o = o;
    a.in_dtype = in_dtype; a.g_dtype = g_dtype; a.o_dtype = o_dtype;
    a.B = B; a.T = T; a.n_seqs = n_seqs; a.H = H; a.dk = dk; a.dv = dv;
    a.head0 = 0; a.heads = H; a.single_stream = single_stream ? 1 : 0;
    a.scale = scale; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.ckpt = ckpt; a.ckpt_every = ckpt_every; a.ckpt_slots = ckpt_slots;
    return from_hip(kda::launch_chunk(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* beta, int in_dtype,
                  const void* g, int g_dtype, const float* initial_state, float* final_state,
                  const int32_t* cu_seqlens, void* o, int o_dtype, int32_t B, int64_t T,
                  int32_t n_seqs, int32_t H, int32_t dk, int32_t dv, int32_t chunk, float scale,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(q, k, v, beta, in_dtype, g, g_dtype, nullptr, 0.0f, initial_state,
                          final_state, cu_seqlens, o, o_dtype, B, T, n_seqs, H, dk, dv, chunk,
                          scale, workspace, workspace_bytes, stream, false);
}

int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* beta,
                        int in_dtype, const float* A, const void* z, int z_dtype, float g_min,
                        const float* initial_state, float* final_state, const int32_t* cu_seqlens,
                        void* o, int o_dtype, int32_t B, int64_t T, int32_t n_seqs, int32_t H,
                        int32_t dk, int32_t dv, int32_t chunk, float scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(q, k, v, beta, in_dtype, z, z_dtype, A, g_min, initial_state,
                          final_state, cu_seqlens, o, o_dtype, B, T, n_seqs, H, dk, dv, chunk,
                          scale, workspace, workspace_bytes, stream, true);
}

int kda_chunk_fwd_gated_noalloc(const void* q, const void* k, const void* v, const void* beta,
                                int in_dtype, const float* A, const void* z, int z_dtype,
                                float g_min, const float* initial_state, float* final_state,
                                const int32_t* cu_seqlens, void* o, int o_dtype, int32_t B,
                                int64_t T, int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                                int32_t chunk, float scale, void* stream) {
    // sizes first: a call whose workspace would not fit is refused before any device work
    if (B < 1 || T < 0 || n_seqs < 1 || H < 1 || !valid_dtype(in_dtype))
        return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_d(dk) || !supported_d(dv) || chunk != 64) return KDA_ERR_UNSUPPORTED;
    const size_t need = kda::chunk_workspace_bytes(n_seqs, int64_t(B) * T, H, dk, dv, in_dtype);
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_address(static_cast<hipStream_t>(stream), &ws);
        if (e != hipSuccess) return KDA_ERR_HIP;
    }
    return chunk_fwd_impl(q, k, v, beta, in_dtype, z, z_dtype, A, g_min, initial_state,
                          final_state, cu_seqlens, o, o_dtype, B, T, n_seqs, H, dk, dv, chunk,
                          scale, ws, need > 0 ? size_t(KDA_NOALLOC_SCRATCH_BYTES) : 0, stream,
                          true, nullptr, 0, 0, /*single_stream=*/true);
}

int kda_chunk_fwd_checkpointed(const void* q, const void* k, const void* v, const void* beta,
                               int in_dtype, const float* A, const void* g_or_z, int gz_dtype,
                               float g_min, const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, void* o, int o_dtype, int32_t B,
                               int64_t T, int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                               int32_t chunk, float scale, float* checkpoints,
                               int32_t checkpoint_every, int64_t max_checkpoints, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (!checkpoints || checkpoint_every < 64 || checkpoint_every % 64 != 0 || max_checkpoints < 0)
        return KDA_ERR_INVALID_ARGUMENT;
    if (B < 1 || T < 0 || n_seqs < 1) return KDA_ERR_INVALID_ARGUMENT;
    // slots the layout can reach: B * floor(T / every), or floor(T / every) + n_seqs when packed
    const int64_t need = cu_seqlens ? T / checkpoint_every + n_seqs : int64_t(B) * (T / checkpoint_every);
    if (max_checkpoints < need) return KDA_ERR_INVALID_ARGUMENT;
    return chunk_fwd_impl(q, k, v, beta, in_dtype, g_or_z, gz_dtype, A, A ? g_min : 0.0f,
                          initial_state, final_state, cu_seqlens, o, o_dtype, B, T, n_seqs, H, dk,
                          dv, chunk, scale, workspace, workspace_bytes, stream, A != nullptr,
                          checkpoints, checkpoint_every, max_checkpoints);
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* beta, int in_dtype,
                    const void* g, int g_dtype, float* state, void* o, int o_dtype, int32_t N,
                    int32_t H, int32_t dk, int32_t dv, float scale, void* stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(g_dtype) || !valid_dtype(o_dtype))
        return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || H < 1 || dk < 1 || dv < 1 || !std::isfinite(scale)) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_d(dk) || !supported_d(dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !beta || !g || !state || !o) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t units = int64_t(N) * H;
    const Range r_o = range(o, units * dv * esize(o_dtype));
    const Range r_s = range(state, units * dk * dv * 4);
    const Range ins[] = {range(q, units * dk * esize(in_dtype)), range(k, units * dk * esize(in_dtype)),
                         range(v, units * dv * esize(in_dtype)), range(beta, units * esize(in_dtype)),
                         range(g, units * dk * esize(g_dtype))};
    for (const Range& x : ins)
        if (overlap(r_o, x) || overlap(r_s, x)) return KDA_ERR_INVALID_ARGUMENT;
    if (overlap(r_o, r_s)) return KDA_ERR_INVALID_ARGUMENT;
    if (kda::debug_validation_enabled()) {
        bool ok = true;
        if (kda::debug_validate(g, g_dtype, int64_t(N) * H * dk, nullptr, 0, 0, static_cast<hipStream_t>(stream), &ok) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (!ok) return KDA_ERR_INVALID_ARGUMENT;
    }
    return from_hip(kda::launch_decode(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N,
                                       H, dk, dv, scale, static_cast<hipStream_t>(stream)));
}

int kda_decode_verify(const void* q, const void* k, const void* v, const void* beta, int in_dtype,
                      const void* g, int g_dtype, const float* state, void* o, int o_dtype,
                      int32_t N, int32_t K, int32_t H, int32_t dk, int32_t dv, float scale,
                      void* stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(g_dtype) || !valid_dtype(o_dtype))
        return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || K < 1 || H < 1 || dk < 1 || dv < 1 || !std::isfinite(scale))
        return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_d(dk) || !supported_d(dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !beta || !g || !state || !o) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t rows = int64_t(N) * K * H;
    const Range r_o = range(o, rows * dv * esize(o_dtype));
    const Range others[] = {range(q, rows * dk * esize(in_dtype)), range(k, rows * dk * esize(in_dtype)),
                            range(v, rows * dv * esize(in_dtype)), range(beta, rows * esize(in_dtype)),
                            range(g, rows * dk * esize(g_dtype)), range(state, int64_t(N) * H * dk * dv * 4)};
    for (const Range& x : others)
        if (overlap(r_o, x)) return KDA_ERR_INVALID_ARGUMENT;
    if (kda::debug_validation_enabled()) {
        bool ok = true;
        if (kda::debug_validate(g, g_dtype, int64_t(N) * K * H * dk, nullptr, 0, 0, static_cast<hipStream_t>(stream), &ok) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (!ok) return KDA_ERR_INVALID_ARGUMENT;
    }
    return from_hip(kda::launch_decode_verify(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype,
                                              N, K, H, dk, dv, scale, static_cast<hipStream_t>(stream)));
}

int kda_decode_commit(const void* q, const void* k, const void* v, const void* beta, int in_dtype,
                      const void* g, int g_dtype, float* state, const int32_t* accepted, int32_t N,
                      int32_t K, int32_t H, int32_t dk, int32_t dv, void* stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(g_dtype)) return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || K < 1 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_d(dk) || !supported_d(dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !beta || !g || !state || !accepted) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t rows = int64_t(N) * K * H;
    const Range r_s = range(state, int64_t(N) * H * dk * dv * 4);
    const Range others[] = {range(q, rows * dk * esize(in_dtype)), range(k, rows * dk * esize(in_dtype)),
                            range(v, rows * dv * esize(in_dtype)), range(beta, rows * esize(in_dtype)),
                            range(g, rows * dk * esize(g_dtype)), range(accepted, int64_t(N) * 4)};
    for (const Range& x : others)
        if (overlap(r_s, x)) return KDA_ERR_INVALID_ARGUMENT;
    if (kda::debug_validation_enabled()) {
        bool ok = true;
        if (kda::debug_validate(g, g_dtype, int64_t(N) * K * H * dk, nullptr, 0, 0, static_cast<hipStream_t>(stream), &ok) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (!ok) return KDA_ERR_INVALID_ARGUMENT;
    }
    return from_hip(kda::launch_decode_commit(q, k, v, beta, in_dtype, g, g_dtype, state, accepted,
                                              N, K, H, dk, dv, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
