/*
 * kda_oracle.c -- plain fp64 CPU reference for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this library: it is
 * used by the test suite, by the smoke check and by the CPU-baseline leg of the benchmark.
 * It shares no code, header, table or helper with the HIP library; it is deliberately slow
 * and obviously correct (one token at a time, every step written out in full, fp64).
 *
 * Pages this follows (titles as published):
 *   [bagrov]  "Архитектура Kimi K3: как открытая модель с миллионным контекстом конкурирует
 *             с лидерами рынка" (bagrov.by)
 *   [habr]    "Как устроена Kimi K3: 2,8 трлн параметров, линейное внимание и агенты на
 *             миллион токенов" (savepearlharbor.com)
 *   [tgstat]  "Kimi K3: Open Frontier Intelligence" (tgstat.ru, @datastorieslanguages)
 *
 * What is computed, per (sequence, head) and token t, with a d_k x d_v state S:
 *   alpha_t = exp(g_t)             (one factor per key channel)
 *   S  <- Diag(alpha_t) S          forget first                      [habr, § Последовательность]
 *   u_t = v_t - S^T k_t            what the state already says about k_t
 *   S  <- S + beta_t k_t u_t^T     overwrite along k_t with strength beta_t
 *                                                        [bagrov, § Как архитектура … миллион токенов]
 *   o_t = scale * S^T q_t          read-out from the updated state
 * Taken together this is S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 * o_t = S_t^T q_t: the state has a fixed size, each token partly erases what is stored along
 * its key and writes its value there ([bagrov] same section; [tgstat] post body, which calls
 * the forget gates channel-wise).  The pages print no formula for the update itself; the
 * reading above (forget applied before the write, output from the post-write state, the
 * forget factor scaling the key axis) is the plainest one consistent with them.
 *
 * Gate ([habr, § Последовательность]): g = g_min * sigmoid(exp(A) * z), alpha = exp(g),
 * g_min = -5, with A one value per (head, key channel) and z one value per (token, head,
 * key channel).  sigmoid(x) = 1 / (1 + exp(-x)).
 *
 * Parity pins for every function here live in tests/ (closed forms, invariants, brute-force
 * transition products); none of them calls this file's formulas a second time.
 *
 * Storage: inputs arrive in their stored dtype and are upcast exactly to double
 * (ORC_F32 = IEEE binary32, ORC_BF16 = upper 16 bits of a binary32, ORC_F64 = binary64).
 * Layouts (row-major): q, k, g, z: [tokens, H, d_k]; v, o: [tokens, H, d_v]; beta: [tokens, H];
 * state: [N, H, d_k, d_v] (key channel = row).  "tokens" is B*T for fixed-length batches
 * (token index b*T + t) or the packed total for variable-length batches (cu_seqlens).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* Exact upcast of element i of a buffer stored as dtype dt. */
static double ld(const void *p, int dt, int64_t i) {
    if (dt == ORC_F32) return (double)((const float *)p)[i];
    if (dt == ORC_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[i];
}

/* Gate: g[t,h,c] = g_min * sigmoid(exp(A[h,c]) * z[t,h,c]). */
void kda_oracle_gate(const void *A, int a_dt, const void *z, int z_dt, double *g,
                     int64_t n_tokens, int H, int dk, double g_min) {
    for (int64_t t = 0; t < n_tokens; ++t)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < dk; ++c) {
                int64_t i = (t * H + h) * dk + c;
                double x = exp(ld(A, a_dt, (int64_t)h * dk + c)) * ld(z, z_dt, i);
                double sig = 1.0 / (1.0 + exp(-x));
                g[i] = g_min * sig;
            }
}

/*
 * One token of the recurrence on a single (sequence, head) state S[dk][dv] (double, in place).
 * qk_off is the element offset of the token's d_k channels in q, k and g, v_off that of its
 * d_v values in v, b_off that of its beta; the output row (d_v doubles) is written to o_row
 * when it is not NULL.  u is scratch of length dv.
 */
static void token_step(double *S, int dk, int dv, const void *q, const void *k, const void *v,
                       const void *beta, const void *g, int in_dt, int g_dt, int64_t qk_off,
                       int64_t v_off, int64_t b_off, double scale, double *u, double *o_row) {
    /* forget: every key-channel row of S is scaled by alpha = exp(g) */
    for (int i = 0; i < dk; ++i) {
        double alpha = exp(ld(g, g_dt, qk_off + i));
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= alpha;
    }
    /* innovation u = v - S^T k */
    for (int j = 0; j < dv; ++j) u[j] = ld(v, in_dt, v_off + j);
    for (int i = 0; i < dk; ++i) {
        double ki = ld(k, in_dt, qk_off + i);
        for (int j = 0; j < dv; ++j) u[j] -= S[i * dv + j] * ki;
    }
    /* write S += beta k u^T */
    double b = ld(beta, in_dt, b_off);
    for (int i = 0; i < dk; ++i) {
        double bk = b * ld(k, in_dt, qk_off + i);
        for (int j = 0; j < dv; ++j) S[i * dv + j] += bk * u[j];
    }
    /* read-out o = scale * S^T q */
    if (o_row) {
        for (int j = 0; j < dv; ++j) o_row[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            double qi = ld(q, in_dt, qk_off + i);
            for (int j = 0; j < dv; ++j) o_row[j] += S[i * dv + j] * qi;
        }
        for (int j = 0; j < dv; ++j) o_row[j] *= scale;
    }
}

/*
 * One (sequence, head) unit over tokens [tok0, tok0 + len) of a [tokens, H, .] batch.
 * S (dk*dv doubles) holds the entering state and receives the final one.
 * o_out, when not NULL, receives len rows of d_v doubles; row r goes to o_out + r*o_tstride.
 */
void kda_oracle_unit(const void *q, const void *k, const void *v, const void *beta, const void *g,
                     int in_dt, int g_dt, int64_t tok0, int64_t len, int H, int h, int dk,
                     int dv, double scale, double *S, double *o_out, int64_t o_tstride) {
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int64_t r = 0; r < len; ++r) {
        int64_t tok = tok0 + r;
        token_step(S, dk, dv, q, k, v, beta, g, in_dt, g_dt, (tok * H + h) * dk,
                   (tok * H + h) * dv, tok * H + h, scale, u, o_out ? o_out + r * o_tstride : NULL);
    }
    free(u);
}

/*
 * Whole batch: every (sequence, head) unit, in parallel over units (they are independent).
 *   cu_seqlens: NULL for B fixed-length sequences of T tokens (n_seqs must equal B), or a
 *               host array of n_seqs+1 offsets into a single packed sequence (B must be 1).
 *   S0: entering states [n_seqs, H, dk, dv] in dtype s0_dt, or NULL for zeros.
 *   o:  [tokens, H, dv] doubles (may be NULL); S_final: [n_seqs, H, dk, dv] doubles (may be NULL).
 *   nthreads <= 0 lets OpenMP choose.  Returns the thread count used.
 */
int kda_oracle_forward(const void *q, const void *k, const void *v, const void *beta, const void *g,
                       int in_dt, int g_dt, const void *S0, int s0_dt, const int32_t *cu_seqlens,
                       double *o, double *S_final, int B, int64_t T, int n_seqs, int H, int dk,
                       int dv, double scale, int nthreads) {
    (void)B;
    int64_t units = (int64_t)n_seqs * H;
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t uidx = 0; uidx < units; ++uidx) {
        int n = (int)(uidx / H), h = (int)(uidx % H);
        int64_t tok0 = cu_seqlens ? cu_seqlens[n] : (int64_t)n * T;
        int64_t len = cu_seqlens ? (int64_t)cu_seqlens[n + 1] - cu_seqlens[n] : T;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        int64_t sbase = uidx * dk * dv;
        for (int64_t e = 0; e < (int64_t)dk * dv; ++e) S[e] = S0 ? ld(S0, s0_dt, sbase + e) : 0.0;
        kda_oracle_unit(q, k, v, beta, g, in_dt, g_dt, tok0, len, H, h, dk, dv, scale, S,
                        o ? o + (tok0 * H + h) * dv : NULL, (int64_t)H * dv);
        if (S_final) memcpy(S_final + sbase, S, sizeof(double) * (size_t)dk * dv);
        free(S);
    }
    return used;
}

/*
 * One decode step for N independent sequences: the same token update applied to each
 * (sequence, head) state in place.  q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H];
 * S: [N, H, dk, dv] doubles (in/out); o: [N, H, dv] doubles (may be NULL).
 */
void kda_oracle_decode_step(const void *q, const void *k, const void *v, const void *beta,
                            const void *g, int in_dt, int g_dt, double *S, double *o, int N, int H,
                            int dk, int dv, double scale, int nthreads) {
    int64_t units = (int64_t)N * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t uidx = 0; uidx < units; ++uidx) {
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        token_step(S + uidx * dk * dv, dk, dv, q, k, v, beta, g, in_dt, g_dt, uidx * dk,
                   uidx * dv, uidx, scale, u, o ? o + uidx * dv : NULL);
        free(u);
    }
}
