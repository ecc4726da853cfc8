// kda_decode.hip -- one-token recurrent update of N independent KDA states, in place.
//
// Pages: "Архитектура Kimi K3: как открытая модель с миллионным контекстом конкурирует с
// лидерами рынка" (bagrov.by), § "Как архитектура Kimi K3 удерживает миллион токенов
// контекста" (fixed-size state, delta-rule overwrite with write strength beta and forget
// factor alpha); "Как устроена Kimi K3: …" (savepearlharbor.com), § "Как обслуживать два
// разных кеша" (the cost of a decode step is reading the large recurrent state).
//
// Per (sequence, head), with alpha = exp(g):
//     a = S^T (alpha * k),  b = S^T (alpha * q)          one read of S, reductions over d_k
//     u = v - a,            o = scale * (b + beta * (k . q) * u)
//     S <- Diag(alpha) S + beta k u^T                     one write of S
// (o follows from o = S_new^T q = S^T Diag(alpha) q + beta u (k . q).)
//
// Speculative decoding, K draft tokens of a sequence on one read of the state: verify returns
// every token's output and leaves the state alone; commit replays the accepted prefix (from the
// same token inputs) and writes the state once.  decode_verify_kernel evaluates drafts of up to 8
// tokens together (projections of the initial state plus one rank-one term per earlier token);
// decode_multi_kernel runs commit and longer drafts token by token with the state in registers.
//
// Layout: one 256-lane workgroup per (sequence, head).  Lane t owns four consecutive state
// columns (16-byte loads/stores) of d_k / (256 / (d_v / 4)) consecutive rows, so each row is
// read by d_v/4 lanes as one contiguous segment.  Partial column sums meet in LDS.  The state
// stays in registers between the read and the write; HBM sees it exactly once each way.  The
// state is streamed with non-temporal loads and stores: a decode step touches each state once,
// so keeping it out of the caches leaves them to the small per-token inputs.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 stream_load4(const float* p) {
    const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void stream_store4(float* p, float4 x) {
    const f32x4_t y = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(y, reinterpret_cast<f32x4_t*>(p));
}

// Shared memory of one step.
template <int DK, int DV>
struct StepSmem {
    static constexpr int CG = DV / 4, RG = 256 / CG;
    float alpha[DK], ak[DK], aq[DK], k[DK];
    float4 red_a[RG][CG];
    float4 red_b[RG][CG];
    float kq[4];
};

// A token's inputs as one lane uses them: lanes t < DK hold channel t of g, k, q; every lane holds
// its four columns of v and beta.  The single-token step loads them before the state read, so its
// token does not wait on a second memory round trip.
struct TokIn {
    float g, k, q, beta;
    float4 v;
};
template <int DK, int DV, int IDT, int GDT>
__device__ __forceinline__ TokIn load_token(const void* __restrict__ q, const void* __restrict__ k,
                                            const void* __restrict__ v, const void* __restrict__ beta,
                                            const void* __restrict__ g, int64_t tok) {
    const int t = threadIdx.x, cg = t % (DV / 4);
    TokIn in;
    in.g = in.k = in.q = 0.f;
    if (t < DK) {
        in.g = load_as_f32<GDT>(g, tok * DK + t);
        in.k = load_as_f32<IDT>(k, tok * DK + t);
        in.q = load_as_f32<IDT>(q, tok * DK + t);
    }
    in.beta = load_as_f32<IDT>(beta, tok);
    in.v = load4_as_f32<IDT>(v, tok * DV + 4 * cg);
    return in;
}

// One token of one (sequence, head) on the state held in registers s[] (rows rg*RPT + i, columns
// 4cg .. 4cg+3), from its inputs `in`; tok indexes its output row, which o (if not null)
// receives.  With STORE each updated row also goes to S as soon as it is formed (interleaving the
// stores with the update keeps the write stream smooth).  Every lane of the workgroup calls it.
template <int DK, int DV, int ODT, bool STORE>
__device__ __forceinline__ void decode_token(float4 (&s)[DK / (256 / (DV / 4))], StepSmem<DK, DV>& sm,
                                             const TokIn& in, int64_t tok, void* __restrict__ o,
                                             float scale, float* __restrict__ S) {
    constexpr int CG = DV / 4;    // lanes per state row
    constexpr int RG = 256 / CG;  // row groups
    constexpr int RPT = DK / RG;  // rows per lane
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;

    float kq = 0.0f;
    if (t < DK) {
        const float a = expf(in.g);
        const float kk = in.k;
        const float qq = in.q;
        sm.alpha[t] = a;
        sm.ak[t] = a * kk;
        sm.aq[t] = a * qq;
        sm.k[t] = kk;
        kq = kk * qq;
    }
    // k . q over the first DK lanes (wavefront reduction, then one value per wave)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off, 64);
    if ((t & 63) == 0) sm.kq[t >> 6] = kq;
    __syncthreads();

    float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg * RPT + i;
        const float ak = sm.ak[r], aq = sm.aq[r];
        pa.x += ak * s[i].x; pa.y += ak * s[i].y; pa.z += ak * s[i].z; pa.w += ak * s[i].w;
        pb.x += aq * s[i].x; pb.y += aq * s[i].y; pb.z += aq * s[i].z; pb.w += aq * s[i].w;
    }
    sm.red_a[rg][cg] = pa;
    sm.red_b[rg][cg] = pb;
    __syncthreads();

    float4 A4 = make_float4(0.f, 0.f, 0.f, 0.f), B4 = A4;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const float4 x = sm.red_a[r][cg], y = sm.red_b[r][cg];
        A4.x += x.x; A4.y += x.y; A4.z += x.z; A4.w += x.w;
        B4.x += y.x; B4.y += y.y; B4.z += y.z; B4.w += y.w;
    }
    const float kqs = sm.kq[0] + sm.kq[1] + sm.kq[2] + sm.kq[3];
    const float bt = in.beta;
    const float4 vv = in.v;
    const float4 u = make_float4(vv.x - A4.x, vv.y - A4.y, vv.z - A4.z, vv.w - A4.w);
    if (o != nullptr && rg == 0) {
        const float c = bt * kqs;
        const float4 oo = make_float4(scale * (B4.x + c * u.x), scale * (B4.y + c * u.y),
                                      scale * (B4.z + c * u.z), scale * (B4.w + c * u.w));
        store4_from_f32<ODT>(o, tok * DV + 4 * cg, oo);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg * RPT + i;
        const float al = sm.alpha[r], bk = bt * sm.k[r];
        s[i].x = al * s[i].x + bk * u.x;
        s[i].y = al * s[i].y + bk * u.y;
        s[i].z = al * s[i].z + bk * u.z;
        s[i].w = al * s[i].w + bk * u.w;
        if constexpr (STORE) stream_store4(S + r * DV + 4 * cg, s[i]);
    }
}

template <int DK, int DV, int IDT, int GDT, int ODT>
__global__ void __launch_bounds__(256) decode_kernel(const void* __restrict__ q,
                                                     const void* __restrict__ k,
                                                     const void* __restrict__ v,
                                                     const void* __restrict__ beta,
                                                     const void* __restrict__ g,
                                                     float* __restrict__ state,
                                                     void* __restrict__ o, float scale) {
    constexpr int CG = DV / 4;    // lanes per state row
    constexpr int RG = 256 / CG;  // row groups
    constexpr int RPT = DK / RG;  // rows per lane
    static_assert(RPT >= 1 && RG * RPT == DK, "shape");
    __shared__ StepSmem<DK, DV> sm;

    const int64_t unit = blockIdx.x;  // sequence * H + head
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    float* S = state + unit * (DK * DV);

    // The token's inputs, then the whole state read.
    const TokIn in = load_token<DK, DV, IDT, GDT>(q, k, v, beta, g, unit);
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = stream_load4(S + (rg * RPT + i) * DV + 4 * cg);
    decode_token<DK, DV, ODT, true>(s, sm, in, unit, o, scale, S);
}

// Several tokens per sequence on one read of the state ([habr, § Как обслуживать два разных
// кеша]: reading the recurrent state is the cost of a decode step).  Tokens are [N, K, H, d]:
// token j of sequence n is row (n*K + j)*H + h.
//   COMMIT = false (verify): all K tokens, o for each, the state is not written.
//   COMMIT = true: the first accepted[n] tokens (clamped to [0, K]), no o, the state written once.
constexpr int MULTI_PRE = 8;     // tokens whose inputs are staged before the state read

template <int DK, int DV, int IDT, int GDT, int ODT, bool COMMIT>
__global__ void __launch_bounds__(256) decode_multi_kernel(const void* __restrict__ q,
                                                           const void* __restrict__ k,
                                                           const void* __restrict__ v,
                                                           const void* __restrict__ beta,
                                                           const void* __restrict__ g,
                                                           float* __restrict__ state,
                                                           void* __restrict__ o, float scale,
                                                           int32_t K, int32_t H,
                                                           const int32_t* __restrict__ accepted) {
    constexpr int CG = DV / 4;
    constexpr int RG = 256 / CG;
    constexpr int RPT = DK / RG;
    static_assert(RPT >= 1 && RG * RPT == DK, "shape");
    __shared__ StepSmem<DK, DV> sm;

    const int64_t unit = blockIdx.x;  // sequence * H + head
    const int64_t n = unit / H, h = unit % H;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    float* S = state + unit * (DK * DV);

    int32_t steps = K;
    if constexpr (COMMIT) {
        const int32_t a = accepted[n];
        steps = a < 0 ? 0 : (a > K ? K : a);
        if (steps == 0) return;                  // nothing accepted: the state stays as it is
    }
    auto tok = [&](int32_t j) -> int64_t { return (n * K + j) * H + h; };

    // The inputs of the first MULTI_PRE tokens are staged in LDS from loads issued before the
    // state read: loads complete in issue order, so inputs loaded after the state would wait for
    // all of it, and each later token for a round trip of its own.  The loads take no branch (the
    // compiler would move them into it, behind the state read): token indices clamp to K - 1 and
    // what the clamped loads bring is never read.  Later tokens load at their start.
    constexpr int PRE = MULTI_PRE, CH = PRE * DK;       // g, k, q of token j, channel c at
    __shared__ __align__(16) float pin[3 * CH];         //   a * CH + j * DK + c (a = 0, 1, 2)
    __shared__ float4 pv[PRE][CG];
    __shared__ float pb[PRE];
    static_assert(CH % 256 == 0, "staging");
    auto tokc = [&](int j) { return tok(j < K ? j : K - 1); };
    // one four-channel group of each of g, k, q per lane (lanes past CH / 4 load a copy)
    const int e4 = t % (CH / 4), j4 = 4 * e4 / DK, c4 = 4 * e4 % DK;
    const float4 xg = load4_as_f32<GDT>(g, tokc(j4) * DK + c4);
    const float4 xk = load4_as_f32<IDT>(k, tokc(j4) * DK + c4);
    const float4 xq = load4_as_f32<IDT>(q, tokc(j4) * DK + c4);
    constexpr int VPL = (PRE * CG + 255) / 256;
    float4 vr[VPL];
#pragma unroll
    for (int p = 0; p < VPL; ++p) {
        const int e = (t + 256 * p) % (PRE * CG);
        vr[p] = load4_as_f32<IDT>(v, tokc(e / CG) * DV + 4 * (e % CG));
    }
    const float br = load_as_f32<IDT>(beta, tokc(t % PRE));

    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = stream_load4(S + (rg * RPT + i) * DV + 4 * cg);

    reinterpret_cast<float4*>(pin)[e4] = xg;          // (lanes past CH / 4 rewrite a copy)
    reinterpret_cast<float4*>(pin + CH)[e4] = xk;
    reinterpret_cast<float4*>(pin + 2 * CH)[e4] = xq;
#pragma unroll
    for (int p = 0; p < VPL; ++p) {
        const int e = (t + 256 * p) % (PRE * CG);       // (lanes past PRE * CG rewrite a copy)
        pv[e / CG][e % CG] = vr[p];
    }
    pb[t % PRE] = br;                                   // (every lane: copies of the same value)
    __syncthreads();

    auto inputs = [&](int32_t j) {
        if (j >= PRE) return load_token<DK, DV, IDT, GDT>(q, k, v, beta, g, tok(j));
        TokIn in;
        in.g = in.k = in.q = 0.f;
        if (t < DK) {
            in.g = pin[j * DK + t];
            in.k = pin[CH + j * DK + t];
            in.q = pin[2 * CH + j * DK + t];
        }
        in.beta = pb[j];
        in.v = pv[j][cg];
        return in;
    };
    const int32_t last = COMMIT ? steps - 1 : steps;   // commit: the last token also stores S
    for (int32_t j = 0; j < last; ++j) {
        if (j > 0) __syncthreads();              // the previous token's shared values are read
        decode_token<DK, DV, ODT, false>(s, sm, inputs(j), tok(j), COMMIT ? nullptr : o, scale, S);
    }
    if constexpr (COMMIT) {
        if (last > 0) __syncthreads();
        decode_token<DK, DV, ODT, true>(s, sm, inputs(last), tok(last), nullptr, scale, S);
    }
}

// Verify from one read of the state, batched over the draft.  With G_j = g_0 + ... + g_j per
// channel, the state before token j satisfies
//     S_j^T y = S_0^T (e^{G_{j-1}} * y) + sum_{i<j} beta_i u_i (k_i . (e^{G_{j-1} - G_i} * y)),
// so token j's a_j = S_j^T (alpha_j * k_j) and b_j = S_j^T (alpha_j * q_j) are
//     a_j = S_0^T (e^{G_j} * k_j) + sum_{i<j} beta_i ck_ji u_i,   ck_ji = sum_d k_i e^{G_j - G_i} k_j
//     b_j = S_0^T (e^{G_j} * q_j) + sum_{i<j} beta_i cq_ji u_i,   cq_ji = sum_d k_i e^{G_j - G_i} q_j
// with u_j = v_j - a_j and o_j = scale (b_j + beta_j (k_j . q_j) u_j).  The 2K projections
// against S_0 are one pass over the state (no per-token pass, no state update); the K x K
// scalars are reductions over d_k; the recurrence for u runs on d_v-vectors.  Token 0 takes
// exactly the step kernel's arithmetic; later tokens equal successive steps up to rounding.
constexpr int VERIFY_KMAX = 8;   // longer drafts run decode_multi_kernel
constexpr int VERIFY_PV = 2;     // projection vectors per pass over the registers

template <int DK, int DV, int IDT, int GDT, int ODT>
__global__ void __launch_bounds__(256) decode_verify_kernel(const void* __restrict__ q,
                                                            const void* __restrict__ k,
                                                            const void* __restrict__ v,
                                                            const void* __restrict__ beta,
                                                            const void* __restrict__ g,
                                                            const float* __restrict__ state,
                                                            void* __restrict__ o, float scale,
                                                            int32_t K, int32_t H) {
    constexpr int CG = DV / 4, RG = 256 / CG, RPT = DK / RG;
    constexpr int KM = VERIFY_KMAX, NV = 2 * KM, NPAIR = KM * (KM - 1) / 2;
    static_assert(RPT >= 1 && RG * RPT == DK && DK <= 256, "shape");
    __shared__ float xv[NV][DK];                  // e^{G_j} k_j at 2j, e^{G_j} q_j at 2j + 1
    __shared__ float4 red[RG][VERIFY_PV][CG];     // partial projections of one pass
    __shared__ float4 tot[NV][CG];                // the projections S_0^T x
    __shared__ float scal[4][2 * NPAIR + KM];     // per-wave partial sums of ck, cq, k.q
    constexpr int VPL = (KM * CG + 255) / 256;   // v chunks per lane
    __shared__ float4 vin[VPL * 256 / CG][CG];    // the draft's v rows (rows >= K unused)
    __shared__ float bin[256];                    // and its betas (entries >= K unused)

    const int64_t unit = blockIdx.x;  // sequence * H + head
    const int64_t n = unit / H, h = unit % H;
    const int t = threadIdx.x, wave = t >> 6;
    const int cg = t % CG, rg = t / CG;
    auto tok = [&](int32_t j) -> int64_t { return (n * K + j) * H + h; };

    // The draft's inputs go out before the state read: loads complete in issue order, so the work
    // on them overlaps the state's arrival instead of waiting for it.  The loads take no branch (a
    // branch would make each wait for its value there): token indices clamp to K - 1 (K >= 1) and
    // what the clamped loads bring for j >= K is never read.  Lane t takes channel t mod DK of g,
    // k and q (lanes t < DK use theirs), v chunk t (+ 256 p) and the beta of token t.
    const int ch = t % DK;
    auto tokc = [&](int j) { return tok(j < K ? j : K - 1); };
    float G[KM], kk[KM], qq[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        G[j] = load_as_f32<GDT>(g, tokc(j) * DK + ch);
        kk[j] = load_as_f32<IDT>(k, tokc(j) * DK + ch);
        qq[j] = load_as_f32<IDT>(q, tokc(j) * DK + ch);
    }
    float4 vr[VPL];
#pragma unroll
    for (int p = 0; p < VPL; ++p) {
        const int e = t + 256 * p;
        vr[p] = load4_as_f32<IDT>(v, tokc(e / CG) * DV + 4 * (e % CG));
    }
    const float br = load_as_f32<IDT>(beta, tokc(t));

    const float* S = state + unit * (DK * DV);
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = stream_load4(S + (rg * RPT + i) * DV + 4 * cg);

    // (stored whole, with no branch, so the compiler keeps the loads ahead of the state read)
#pragma unroll
    for (int p = 0; p < VPL; ++p) {
        const int e = t + 256 * p;
        vin[e / CG][e % CG] = vr[p];
    }
    bin[t] = br;

    // channel ch: cumulative log decays, the projection vectors, and the scalars summed over the
    // channels (pair index p = j (j - 1) / 2 + i for i < j).  Every wave computes (waves past the
    // first DK lanes on a copy of the channels) and only lanes t < DK store: a branch around the
    // work would let the compiler move the input loads into it, behind the state read.
    auto wsum = [&](float r) {
        // no fused multiply-add of the caller's product into the first add: the product rounds
        // first, as in the step kernel, so token 0's k . q matches it bit for bit
#pragma clang fp contract(off)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) r += __shfl_xor(r, off, 64);
        return r;
    };
    const bool owner = t < DK;
    {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            acc += G[j];
            G[j] = acc;
            const float e = expf(acc);
            if (owner) {
                xv[2 * j][t] = e * kk[j];
                xv[2 * j + 1][t] = e * qq[j];
            }
        }
        const bool lead = owner && (t & 63) == 0;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (j >= K) break;
            const float kq = wsum(kk[j] * qq[j]);
            if (lead) scal[wave][2 * NPAIR + j] = kq;
#pragma unroll
            for (int i = 0; i < j; ++i) {
                const int pi = j * (j - 1) / 2 + i;
                const float w = kk[i] * expf(G[j] - G[i]);
                const float ck = wsum(w * kk[j]), cq = wsum(w * qq[j]);
                if (lead) {
                    scal[wave][pi] = ck;
                    scal[wave][NPAIR + pi] = cq;
                }
            }
        }
    }
    __syncthreads();

    // the projections, VERIFY_PV vectors a pass: partial sums over this lane's rows, then over
    // the row groups
    const int NVK = 2 * K;
    for (int v0 = 0; v0 < NVK; v0 += VERIFY_PV) {
        if (v0 > 0) __syncthreads();             // the previous pass's partials are read
#pragma unroll
        for (int w = 0; w < VERIFY_PV; ++w) {
            float4 pa = make_float4(0.f, 0.f, 0.f, 0.f);
            if (v0 + w < NVK) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const float x = xv[v0 + w][rg * RPT + i];
                    pa.x += x * s[i].x; pa.y += x * s[i].y; pa.z += x * s[i].z; pa.w += x * s[i].w;
                }
            }
            red[rg][w][cg] = pa;
        }
        __syncthreads();
        if (t < VERIFY_PV * CG) {                // lane (w, c) sums vector v0 + w over the row groups
            const int w = t / CG, c = t % CG;
            float4 A4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const float4 x = red[r][w][c];
                A4.x += x.x; A4.y += x.y; A4.z += x.z; A4.w += x.w;
            }
            if (v0 + w < NVK) tot[v0 + w][c] = A4;
        }
    }
    __syncthreads();

    // the tokens in order, lane c of the first row group owning columns 4c .. 4c + 3; a scalar is
    // the sum of the channel-holding waves' partials in wave order (token 0's k . q as the step
    // kernel sums it)
    auto csum = [&](int x) {
        float r = scal[0][x];
#pragma unroll
        for (int w = 1; w < (DK + 63) / 64; ++w) r += scal[w][x];
        return r;
    };
    if (t < CG) {
        float4 u[KM];
        float bt[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (j >= K) break;
            bt[j] = bin[j];
            const float4 vv = vin[j][t];
            float4 a = tot[2 * j][t], b = tot[2 * j + 1][t];
#pragma unroll
            for (int i = 0; i < j; ++i) {
                const int pi = j * (j - 1) / 2 + i;
                const float ck = bt[i] * csum(pi), cq = bt[i] * csum(NPAIR + pi);
                a.x += ck * u[i].x; a.y += ck * u[i].y; a.z += ck * u[i].z; a.w += ck * u[i].w;
                b.x += cq * u[i].x; b.y += cq * u[i].y; b.z += cq * u[i].z; b.w += cq * u[i].w;
            }
            u[j] = make_float4(vv.x - a.x, vv.y - a.y, vv.z - a.z, vv.w - a.w);
            const float c = bt[j] * csum(2 * NPAIR + j);
            const float4 oo = make_float4(scale * (b.x + c * u[j].x), scale * (b.y + c * u[j].y),
                                          scale * (b.z + c * u[j].z), scale * (b.w + c * u[j].w));
            store4_from_f32<ODT>(o, tok(j) * DV + 4 * t, oo);
        }
    }
}

template <int DK, int DV, int IDT, int GDT, int ODT>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* beta,
                                  const void* g, float* state, void* o, int32_t N, int32_t H,
                                  float scale, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(N) * H;
    hipLaunchKernelGGL((decode_kernel<DK, DV, IDT, GDT, ODT>), dim3(static_cast<unsigned>(units)),
                       dim3(256), 0, stream, q, k, v, beta, g, state, o, scale);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t dispatch_dtypes(const void* q, const void* k, const void* v, const void* beta,
                                  int idt, const void* g, int gdt, float* state, void* o, int odt,
                                  int32_t N, int32_t H, float scale, hipStream_t s) {
#define KDA_DEC(I, G, O)                                                                       \
    if (idt == I && gdt == G && odt == O)                                                      \
        return launch_decode_t<DK, DV, I, G, O>(q, k, v, beta, g, state, o, N, H, scale, s);
    KDA_DEC(KDA_BF16, KDA_BF16, KDA_BF16)
    KDA_DEC(KDA_BF16, KDA_BF16, KDA_F32)
    KDA_DEC(KDA_BF16, KDA_F32, KDA_BF16)
    KDA_DEC(KDA_BF16, KDA_F32, KDA_F32)
    KDA_DEC(KDA_F32, KDA_BF16, KDA_BF16)
    KDA_DEC(KDA_F32, KDA_BF16, KDA_F32)
    KDA_DEC(KDA_F32, KDA_F32, KDA_BF16)
    KDA_DEC(KDA_F32, KDA_F32, KDA_F32)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

template <int DK, int DV, bool COMMIT>
static hipError_t dispatch_multi(const void* q, const void* k, const void* v, const void* beta,
                                 int idt, const void* g, int gdt, float* state, void* o, int odt,
                                 int32_t N, int32_t K, int32_t H, float scale,
                                 const int32_t* accepted, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(N) * H));
#define KDA_DM(I, G, O)                                                                        \
    if (idt == I && gdt == G && odt == O) {                                                    \
        if (!COMMIT && K <= VERIFY_KMAX)                                                       \
            hipLaunchKernelGGL((decode_verify_kernel<DK, DV, I, G, O>), grid, dim3(256), 0, st, \
                               q, k, v, beta, g, state, o, scale, K, H);                        \
        else                                                                                   \
            hipLaunchKernelGGL((decode_multi_kernel<DK, DV, I, G, O, COMMIT>), grid, dim3(256), \
                               0, st, q, k, v, beta, g, state, o, scale, K, H, accepted);       \
        return hipGetLastError();                                                              \
    }
    KDA_DM(KDA_BF16, KDA_BF16, KDA_BF16)
    KDA_DM(KDA_BF16, KDA_BF16, KDA_F32)
    KDA_DM(KDA_BF16, KDA_F32, KDA_BF16)
    KDA_DM(KDA_BF16, KDA_F32, KDA_F32)
    KDA_DM(KDA_F32, KDA_BF16, KDA_BF16)
    KDA_DM(KDA_F32, KDA_BF16, KDA_F32)
    KDA_DM(KDA_F32, KDA_F32, KDA_BF16)
    KDA_DM(KDA_F32, KDA_F32, KDA_F32)
#undef KDA_DM
    return hipErrorInvalidValue;
}

template <bool COMMIT>
static hipError_t launch_multi(const void* q, const void* k, const void* v, const void* beta,
                               int in_dtype, const void* g, int g_dtype, float* state, void* o,
                               int o_dtype, int32_t N, int32_t K, int32_t H, int32_t dk, int32_t dv,
                               float scale, const int32_t* accepted, hipStream_t s) {
    if (dk == 128 && dv == 128)
        return dispatch_multi<128, 128, COMMIT>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, K, H, scale, accepted, s);
    if (dk == 128 && dv == 64)
        return dispatch_multi<128, 64, COMMIT>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, K, H, scale, accepted, s);
    if (dk == 64 && dv == 128)
        return dispatch_multi<64, 128, COMMIT>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, K, H, scale, accepted, s);
    return dispatch_multi<64, 64, COMMIT>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, K, H, scale, accepted, s);
}

hipError_t launch_decode_verify(const void* q, const void* k, const void* v, const void* beta,
                                int in_dtype, const void* g, int g_dtype, const float* state,
                                void* o, int o_dtype, int32_t N, int32_t K, int32_t H, int32_t dk,
                                int32_t dv, float scale, hipStream_t stream) {
    return launch_multi<false>(q, k, v, beta, in_dtype, g, g_dtype, const_cast<float*>(state), o,
                               o_dtype, N, K, H, dk, dv, scale, nullptr, stream);
}

hipError_t launch_decode_commit(const void* q, const void* k, const void* v, const void* beta,
                                int in_dtype, const void* g, int g_dtype, float* state,
                                const int32_t* accepted, int32_t N, int32_t K, int32_t H,
                                int32_t dk, int32_t dv, hipStream_t stream) {
    // o is not written in commit mode; its dtype only selects an instantiation
    return launch_multi<true>(q, k, v, beta, in_dtype, g, g_dtype, state, nullptr, KDA_F32, N, K,
                              H, dk, dv, 1.0f, accepted, stream);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* beta,
                         int in_dtype, const void* g, int g_dtype, float* state, void* o,
                         int o_dtype, int32_t N, int32_t H, int32_t dk, int32_t dv, float scale,
                         hipStream_t stream) {
    if (dk == 128 && dv == 128)
        return dispatch_dtypes<128, 128>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, H, scale, stream);
    if (dk == 128 && dv == 64)
        return dispatch_dtypes<128, 64>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, H, scale, stream);
    if (dk == 64 && dv == 128)
        return dispatch_dtypes<64, 128>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, H, scale, stream);
    return dispatch_dtypes<64, 64>(q, k, v, beta, in_dtype, g, g_dtype, state, o, o_dtype, N, H, scale, stream);
}

}  // namespace kda
