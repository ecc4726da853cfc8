/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) implementation of the Kimi Delta Attention
 * (KDA) forward pass: the forget gate, chunked prefill and the single-token decode step.
 *
 * Pages the operations come from (titles as published):
 *   [bagrov] "Архитектура Kimi K3: как открытая модель с миллионным контекстом конкурирует с
 *            лидерами рынка" (bagrov.by)
 *   [habr]   "Как устроена Kimi K3: 2,8 трлн параметров, линейное внимание и агенты на миллион
 *            токенов" (savepearlharbor.com)
 *
 * The recurrence, per (sequence, head), with a fixed d_k x d_v state S (key channel = row):
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t,
 *     alpha_t = exp(g_t) (one factor per key channel).
 * The state has a fixed size, each token partly erases what is stored along its key and writes
 * its value there, with write strength beta and forget factor alpha ([bagrov, § Как архитектура
 * Kimi K3 удерживает миллион токенов контекста]); the forget is per channel and acts before
 * the write ([habr, § Последовательность: три KDA на один глобальный MLA]).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE memory owned by the caller; the library keeps no pointer
 *     after returning and allocates no device memory.
 *   - Tensors are contiguous, row-major:
 *       q, k, g, z : [B, T, H, d_k]          v, o : [B, T, H, d_v]          beta : [B, T, H]
 *       state      : [N, H, d_k, d_v] fp32 (row = key channel, d_v contiguous)
 *     Packed variable-length batches use B = 1, T = total tokens and device cu_seqlens[N+1].
 *     The decode step drops T.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream).  There is no host synchronisation and the host never reads device data.
 *     Buffers must stay alive until the stream has passed the work.  Segmented 16-bit prefills
 *     at d_k = d_v = 128 also run half of the heads on a second stream the library keeps per
 *     device (created on first use, never destroyed).  That stream starts after the work already
 *     on `stream` and `stream` waits for it before its next work, so the call's ordering on
 *     `stream` is as for a single stream.  kda_chunk_fwd_gated_noalloc never uses it.
 *   - Every call returns a kda_status; nothing is printed and nothing aborts.  Host-checkable
 *     argument errors are reported before any device work is enqueued.  Device-resident
 *     preconditions (g in [-5, 0], well-formed cu_seqlens) are the caller's contract and are not
 *     checked; violating them gives unspecified results but no out-of-bounds access: the
 *     kernels clamp every offset to 0 <= cu_seqlens[n] <= cu_seqlens[n+1] <= T before using it.
 *   - Debug check: with the environment variable KDA_DEBUG_VALIDATE set (to anything but "" or
 *     "0"), kda_chunk_fwd, kda_chunk_fwd_checkpointed and the three decode calls first test those
 *     preconditions on the device (kda_chunk_fwd_gated tests cu_seqlens only: its g is in range
 *     by construction), wait for the answer on `stream` and return KDA_ERR_INVALID_ARGUMENT,
 *     with nothing else enqueued, on a violation.  This synchronises the host, shares one word
 *     of library-owned device memory between all calls on a device (overlapping checked calls
 *     race on it) and must not be used under stream capture.
 *   - Calls are stateless and reentrant (the debug check aside).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad dtype, aliasing     */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented: d_k/d_v not in {64,128}, ... */
    KDA_ERR_WORKSPACE = 3,        /* workspace smaller than kda_chunk_fwd_workspace_size()   */
    KDA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed              */
} kda_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *kda_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

/*
 * kda_gate -- forget-gate log-decay, [habr, § Последовательность]:
 *     g[t,h,c] = g_min * sigmoid(exp(A[h,c]) * z[t,h,c]),   sigmoid(x) = 1 / (1 + exp(-x)),
 * so alpha = exp(g) lies in [e^g_min, 1].  The pages fix g_min = -5; this bound is what keeps
 * every causal 16-token block of the chunked prefill inside the bf16/fp32 exponent range.
 *   A       : [H, d_k] fp32, device.
 *   z       : [n_tokens, H, d_k] in z_dtype (KDA_F32 or KDA_BF16), device.
 *   g       : [n_tokens, H, d_k] in g_dtype (KDA_F32 or KDA_BF16, round-to-nearest-even), device;
 *             must not overlap z or A.
 *   n_tokens: >= 0 (0 is a no-op); H, d_k >= 1.
 *   g_min   : must lie in [-5, 0); other values return KDA_ERR_UNSUPPORTED.
 * Precision (fp32 g): within 1.5 ulp of the exact value wherever |exp(A) z| <= 126 ln 2 (the
 * hardware exp2 of the rounded argument, 1 ulp, and a corrected quotient, 0.5 ulp; the argument's
 * rounding error is carried separately); beyond that g is g_min or below 2^-123 in magnitude.
 * z = 0 gives g_min / 2 exactly.  bf16 g is the fp32 value rounded.
 */
int kda_gate(const float *A, const void *z, int z_dtype, void *g, int g_dtype, int64_t n_tokens,
             int32_t H, int32_t dk, float g_min, void *stream);

/*
 * Workspace bytes kda_chunk_fwd needs for a batch of n_seqs sequences holding total_tokens tokens
 * (B*T for fixed-length batches) with inputs in in_dtype.  The prefill runs in two kernels: the
 * first computes, for every (head, 32-token record; 16 tokens for fp32 inputs), everything that
 * does not depend on the state and writes it to the workspace; the second passes the state
 * along each sequence reading it.  At d_k = 128 a record is 27.5 KiB for bf16 inputs (880 bytes
 * per token and head) and 26.5 KiB for fp32 inputs (16 tokens).  Long sequences with few
 * (sequence, head) units also need per-segment state buffers.  Batches of bf16 inputs at
 * d_k = d_v = 128 with n_seqs * H >= 256 run one fused kernel that builds the records on chip:
 * their size is 0 (a NULL workspace is accepted).
 * Never fails; returns 0 for invalid sizes (kda_chunk_fwd then reports the error).
 */
size_t kda_chunk_fwd_workspace_size(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dk,
                                    int32_t dv, int32_t chunk, int in_dtype);

/*
 * kda_chunk_fwd -- chunked prefill of the recurrence above over whole sequences.
 * Tokens inside a chunk are handled together and the state is carried from chunk to chunk
 * ([bagrov, § Уровень чипа: специализированное ядро FlashKDA]); with g >= -5 every causal
 * 16-token block, diagonal ones included, is a dense matrix product
 * ([habr, § Последовательность]).
 *   q, k, v, beta : inputs in in_dtype (KDA_F32 or KDA_BF16), layouts above.
 *   g             : [B, T, H, d_k] log-decay in g_dtype (KDA_F32 recommended; KDA_BF16 allowed),
 *                   values must lie in [-5, 0] (caller contract).
 *   initial_state : [N, H, d_k, d_v] fp32 or NULL (= zeros); never written unless it is also
 *                   final_state.
 *   final_state   : [N, H, d_k, d_v] fp32 or NULL; may equal initial_state (in-place update)
 *                   but must not partially overlap it.
 *   cu_seqlens    : NULL for B fixed-length sequences of T tokens (then n_seqs must equal B), or
 *                   device int32 [n_seqs + 1] offsets of a packed batch (then B must be 1,
 *                   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[n_seqs] = T; caller contract).
 *                   Empty sequences are allowed: their final state is their initial state.
 *   o             : [B, T, H, d_v] in o_dtype (KDA_F32 or KDA_BF16); must not overlap any input.
 *   T             : >= 0 (T = 0 only copies initial_state to final_state, or zeroes it).
 *   dk, dv        : 64 or 128 each.  chunk: must be 64.  scale: any finite value (1 = none).
 *   workspace     : device buffer of at least kda_chunk_fwd_workspace_size(...) bytes, owned
 *                   by the caller; its contents on entry do not matter and on return are
 *                   unspecified.  It must not overlap any other argument.  Calls that share
 *                   a workspace must not overlap in time.
 * Results match the token-by-token definition up to rounding: the kernels evaluate the chunked
 * form with fp32 accumulation and split-precision matrix products.  Any finite input values are
 * accepted (beta included: the pages give it no range).  For bf16 inputs the state-pass operands
 * are staged in fp16, whose largest value is 65504: the results hold their tolerance while the
 * state, initial_state, v, scale * |q| * |k| and the entries of each 16-token block's UT
 * transform stay well inside that range.  The usual KDA inputs (q, k L2-normalised, beta in
 * [0, 1], the gate's decay) keep them below 10; the tests also cover beta in [-0.5, 1.5],
 * |q| = |k| = 3 with scale 4 and |v| about 30 (states to about 1000).  Keys with
 * beta * |k|^2 > 2 make the recurrence itself expansive along k (the transition scales that
 * direction by 1 - beta |k|^2 alpha), so long sequences of such inputs overflow any precision.
 * fp32 inputs use bf16 hi/lo splits throughout and have the fp32 range.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *beta, int in_dtype,
                  const void *g, int g_dtype, const float *initial_state, float *final_state,
                  const int32_t *cu_seqlens, void *o, int o_dtype, int32_t B, int64_t T,
                  int32_t n_seqs, int32_t H, int32_t dk, int32_t dv, int32_t chunk, float scale,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd_gated -- kda_chunk_fwd with the forget gate fused in: takes the gate's inputs
 * A [H, d_k] fp32 and z [B, T, H, d_k] (z_dtype KDA_F32 or KDA_BF16) instead of g, and computes
 * g = g_min * sigmoid(exp(A) * z) on the fly ([habr, § Последовательность]) with the same
 * arithmetic as kda_gate, so that g never travels through memory.  The results equal
 * kda_gate followed by kda_chunk_fwd on an fp32 g bit for bit.  g_min must lie in [-5, 0)
 * (KDA_ERR_UNSUPPORTED otherwise); A and z must not overlap o, final_state or the workspace.
 * Every other argument, the workspace size and the error behaviour are those of kda_chunk_fwd.
 */
int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const void *beta,
                        int in_dtype, const float *A, const void *z, int z_dtype, float g_min,
                        const float *initial_state, float *final_state, const int32_t *cu_seqlens,
                        void *o, int o_dtype, int32_t B, int64_t T, int32_t n_seqs, int32_t H,
                        int32_t dk, int32_t dv, int32_t chunk, float scale, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd_gated_noalloc -- kda_chunk_fwd_gated for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It takes no workspace argument; the prefill's workspace is a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES inside the library, which each GPU holds from the first call on it
 * until the process ends.  The call itself allocates nothing.
 *   Sizes: the call is refused with KDA_ERR_WORKSPACE, before any device work, when
 *   kda_chunk_fwd_workspace_size(n_seqs, B*T, H, dk, dv, 64, in_dtype) exceeds
 *   KDA_NOALLOC_SCRATCH_BYTES (256 MiB: e.g. 16-bit inputs with d_k = 128 up to about 290 K
 *   token-heads, such as 4 x 4096 tokens x 16 heads).
 *   Sharing: every call on one GPU uses that GPU's array.  Nothing in it has to start at zero and
 *   it keeps the last call's contents; calls that overlap in time on one GPU (another stream,
 *   another thread) race on it and must be serialised by the caller.
 *   Device: the array of the device `stream` belongs to (the current device for NULL) is used.
 * Every other argument, the results (equal to kda_chunk_fwd_gated's bit for bit) and the error
 * behaviour are those of kda_chunk_fwd_gated.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int kda_chunk_fwd_gated_noalloc(const void *q, const void *k, const void *v, const void *beta,
                                int in_dtype, const float *A, const void *z, int z_dtype,
                                float g_min, const float *initial_state, float *final_state,
                                const int32_t *cu_seqlens, void *o, int o_dtype, int32_t B,
                                int64_t T, int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                                int32_t chunk, float scale, void *stream);

/*
 * kda_chunk_fwd_checkpointed -- the chunked prefill that also stores the state at fixed token
 * boundaries, for prefix caching: a later request that shares a prefix resumes from the stored
 * state (copy it, then continue) instead of recomputing the prefix ([habr, § Как обслуживать
 * два разных кеша]: the recurrent state is what such a cache keeps).
 *   A, g_or_z, gz_dtype, g_min : A non-NULL fuses the gate as kda_chunk_fwd_gated does (g_or_z
 *                   is z, g_min as there); A NULL makes g_or_z the log-decay g of kda_chunk_fwd
 *                   (g_min is then ignored).
 *   checkpoints   : fp32 device buffer [max_checkpoints, H, d_k, d_v] owned by the caller.
 *                   Checkpoint j >= 1 of sequence n is its state after its first
 *                   j * checkpoint_every tokens, for every j with j * checkpoint_every <= len_n
 *                   (the last one equals the final state when the length is a multiple); it goes
 *                   to slot base(n) + j - 1 with base(n) = n * floor(T / checkpoint_every) for
 *                   fixed-length batches and floor(cu_seqlens[n] / checkpoint_every) + n for
 *                   packed ones.  Slots no checkpoint maps to are left untouched.
 *   checkpoint_every : tokens between checkpoints, a positive multiple of 64 (the chunk).
 *   max_checkpoints  : slots in `checkpoints`; at least B * floor(T / checkpoint_every) for
 *                   fixed-length batches and floor(T / checkpoint_every) + n_seqs for packed ones.
 * A NULL buffer, a checkpoint_every that is not a positive multiple of 64, too few slots, or a
 * buffer that overlaps any other argument return KDA_ERR_INVALID_ARGUMENT.  Every other argument,
 * the workspace size and the error behaviour are those of kda_chunk_fwd; o and final_state equal
 * kda_chunk_fwd's (or kda_chunk_fwd_gated's) bit for bit.
 */
int kda_chunk_fwd_checkpointed(const void *q, const void *k, const void *v, const void *beta,
                               int in_dtype, const float *A, const void *g_or_z, int gz_dtype,
                               float g_min, const float *initial_state, float *final_state,
                               const int32_t *cu_seqlens, void *o, int o_dtype, int32_t B,
                               int64_t T, int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                               int32_t chunk, float scale, float *checkpoints,
                               int32_t checkpoint_every, int64_t max_checkpoints, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * kda_decode_step -- one token of the recurrence for N independent sequences, updating each
 * state in place.  One pass reads S once and writes it once: reading the large recurrent
 * state is this step's cost ([habr, § Как обслуживать два разных кеша]).
 *   q, k, g : [N, H, d_k]; v : [N, H, d_v]; beta : [N, H]; q, k, v, beta in in_dtype, g in g_dtype
 *             (KDA_F32 or KDA_BF16 each); g must lie in [-5, 0] (caller contract).
 *   state   : [N, H, d_k, d_v] fp32, read and overwritten in place.
 *   o       : [N, H, d_v] in o_dtype; must not overlap any input or the state.
 *   N >= 0 (0 is a no-op); H >= 1; dk, dv: 64 or 128 each.
 */
int kda_decode_step(const void *q, const void *k, const void *v, const void *beta, int in_dtype,
                    const void *g, int g_dtype, float *state, void *o, int o_dtype, int32_t N,
                    int32_t H, int32_t dk, int32_t dv, float scale, void *stream);

/*
 * Speculative decoding ([habr, § Как обслуживать два разных кеша]: no copy of the state is kept
 * per draft token; the accepted stretch is recomputed on chip from the token inputs, which is
 * cheaper than reading the large state again and again).  A draft of K tokens per sequence is
 * laid out like a prefill batch: q, k, g [N, K, H, d_k]; v [N, K, H, d_v]; beta [N, K, H]
 * (token j of sequence n is row (n*K + j)*H + h).
 *
 * kda_decode_verify -- runs all K draft tokens of every sequence from `state` (read only, never
 * written) and writes each token's output o [N, K, H, d_v] (o_dtype): the outputs K calls of
 * kda_decode_step would give, with one read of the state instead of K reads and writes.  Drafts
 * of up to 8 tokens are evaluated together from one pass over the state (the state after token
 * j is S_0 under the cumulative decay plus j rank-one terms); the first token's output equals
 * kda_decode_step's bit for bit, the others equal it up to fp32 rounding.  Longer drafts run
 * token by token and equal the step outputs bit for bit.  o must not overlap any other argument.
 *
 * kda_decode_commit -- once the draft has been checked, advances each state in place by its
 * accepted tokens: accepted is a device int32 [N] array of counts (values outside [0, K] are
 * clamped; 0 leaves the state untouched).  The same inputs are passed again; no o is produced.  The new
 * state equals accepted[n] successive kda_decode_step calls bit for bit.  The state must not
 * overlap any input or `accepted`.
 *
 * Both: dtypes, dimensions (d_k, d_v in {64, 128}), N >= 0 (0 is a no-op), K >= 1, H >= 1 and the
 * error behaviour as in kda_decode_step; the caller owns every buffer; work is enqueued on
 * `stream`.
 */
int kda_decode_verify(const void *q, const void *k, const void *v, const void *beta, int in_dtype,
                      const void *g, int g_dtype, const float *state, void *o, int o_dtype,
                      int32_t N, int32_t K, int32_t H, int32_t dk, int32_t dv, float scale,
                      void *stream);

int kda_decode_commit(const void *q, const void *k, const void *v, const void *beta, int in_dtype,
                      const void *g, int g_dtype, float *state, const int32_t *accepted, int32_t N,
                      int32_t K, int32_t H, int32_t dk, int32_t dv, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
