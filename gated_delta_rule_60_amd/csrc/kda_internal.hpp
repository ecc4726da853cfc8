// kda_internal.hpp -- launchers the C ABI layer calls after it has validated the arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

hipError_t launch_gate(const float* A, const void* z, int z_dtype, void* g, int g_dtype,
                       int64_t n_tokens, int32_t H, int32_t dk, float g_min, hipStream_t stream);

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* beta,
                         int in_dtype, const void* g, int g_dtype, float* state, void* o,
                         int o_dtype, int32_t N, int32_t H, int32_t dk, int32_t dv, float scale,
                         hipStream_t stream);

// Several tokens per sequence ([N, K, H, d] inputs) on one read of the state: verify writes
// o [N, K, H, dv] and leaves the state; commit applies the first accepted[n] tokens in place.
hipError_t launch_decode_verify(const void* q, const void* k, const void* v, const void* beta,
                                int in_dtype, const void* g, int g_dtype, const float* state,
                                void* o, int o_dtype, int32_t N, int32_t K, int32_t H, int32_t dk,
                                int32_t dv, float scale, hipStream_t stream);
hipError_t launch_decode_commit(const void* q, const void* k, const void* v, const void* beta,
                                int in_dtype, const void* g, int g_dtype, float* state,
                                const int32_t* accepted, int32_t N, int32_t K, int32_t H,
                                int32_t dk, int32_t dv, hipStream_t stream);

// Optional debug check (KDA_DEBUG_VALIDATE): g (g_elems values, or none) within [-5, 0] and, for
// packed batches, cu_seqlens well formed.  Synchronises the stream; *ok = false on a violation.
bool debug_validation_enabled();
hipError_t debug_validate(const void* g, int g_dtype, int64_t g_elems, const int32_t* cu,
                          int32_t n_seqs, int64_t total, hipStream_t stream, bool* ok);

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const void* g;         // log-decay g, or z when the gate is fused (gate_A != nullptr)
    const float* gate_A;   // fused gate: A [H, dk] fp32; nullptr when g is given
    float g_min;           // fused gate: g = g_min * sigmoid(exp(A) * z)
    const float* h0;       // initial state or nullptr
    float* hT;             // final state or nullptr
    const int32_t* cu;     // device cu_seqlens or nullptr
    void* o;
    int in_dtype, g_dtype, o_dtype;   // g_dtype is z's dtype when the gate is fused
    int32_t B;
    int64_t T;
    int32_t n_seqs, H, dk, dv;
    int32_t head0, heads;  // the launch covers heads [head0, head0 + heads); H stays the head
                           // count of every [.., H, ..] layout (a whole call: 0 and H)
    int32_t single_stream; // run on the caller's stream only: no stream or event is created
    float scale;
    void* workspace;
    size_t workspace_bytes;
    float* ckpt;           // state checkpoints or nullptr
    int32_t ckpt_every;    // tokens between checkpoints (a multiple of 64)
    int64_t ckpt_slots;    // capacity of ckpt in [H, dk, dv] states
};

// Segment buffers of a prefill that runs long sequences in segments (see kda_chunk_util.hpp):
// per (segment slot, head) the segment's start state S, its transition M and its zero-start
// state B, fp32.
struct SegArgs {
    float* S;            // [slots, H, d_k, d_v] segment start states
    float* M;            // [slots, H, d_k, d_k]
    float* B;            // [slots, H, d_k, d_v]
    int64_t slots;
    int32_t n_vblk_m;    // column blocks of M (d_k columns) in segment pass 1
    int32_t seg_shift;   // log2 of the segment length in tokens
    int32_t from0;       // pairs start at segment 0 (pass 1 runs pairs only; the scan starts from
                         // the initial state and pass 2 runs every segment); else segment 0 runs
                         // whole in pass 1 and the pairs start at segment 1
};

// Workspace bytes of a chunked prefill (records and/or segment buffers, by path).
size_t chunk_workspace_bytes(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dk,
                             int32_t dv, int32_t in_dtype);

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream);

// The fused kernel (kda_fused.hip): 16-bit inputs at d_k = d_v = 128 with at least 256
// (sequence, head) units -- whole sequences, records built and consumed in LDS, no workspace.
bool fused_eligible(int32_t in_dtype, int32_t dk, int32_t dv, int32_t n_seqs, int32_t H);
hipError_t launch_fused(const ChunkArgs& a, hipStream_t stream);

}  // namespace kda
