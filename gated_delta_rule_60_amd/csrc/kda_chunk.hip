// kda_chunk.hip -- chunked KDA prefill on gfx950: one fused kernel per call.
//
// Pages (titles as published):
//   [bagrov] "Архитектура Kimi K3: как открытая модель с миллионным контекстом конкурирует с
//            лидерами рынка" (bagrov.by): § "Как архитектура Kimi K3 удерживает миллион токенов
//            контекста" (state, delta rule, bounded forget factor), § "Уровень чипа:
//            специализированное ядро FlashKDA" (tokens of a block in parallel, then the state is
//            passed on, spread over independent heads).
//   [habr]   "Как устроена Kimi K3: …" (savepearlharbor.com), § "Последовательность: три KDA на
//            один глобальный MLA" (g = g_min*sigmoid(exp(A) z), g_min = -5 keeps the running decay
//            products inside the bf16 range so every causal 16-token block, diagonal ones included,
//            is a dense matrix product).
//
// Chunk form (derived from the token recurrence; C = 64 tokens, chunk-entering state S):
//   G_r = sum_{t<=r} g_t (per channel),  Kt = e^G * K,  Qt = e^G * Q,  Kb = e^{G_n - G} * K
//   A[r,s] = beta_r sum_c k_rc k_sc e^{G_rc - G_sc}  (s < r),   P[r,s] = sum_c q_rc k_sc e^{G_rc - G_sc} (s <= r)
//   W = (I + A)^{-1} beta*(V - Kt S)          (row r of W is beta_r times token r's innovation)
//   O = scale * (Qt S + P W),                 S <- Diag(e^{G_n}) S + Kb^T W
//
// A and P are built per 16-row block b with the token before the block as reference R_b:
//   diagonal tile:   (k_r e^{G_r - R_b}) . (k_s e^{R_b - G_s})       column factors in [1, e^80]
//   tile b x j<b:    (k_r e^{G_r - R_b} e^{R_b - R_{j+1}}) . (k_s e^{R_{j+1} - G_s})   all factors <= 1
// With g >= -5 a 16-token span decays by at most e^-80, so e^80 < bf16/fp32 max (e^88.7): the
// diagonal tiles are plain dense MFMA tiles (split bf16 for range), no pairwise special case.
//
// Work split: one 256-lane workgroup per (sequence, head, block of 64 state columns).  Each of the
// four waves owns 16 state columns for the whole sequence, in fp32 MFMA accumulators.  Per chunk:
//   staging    lanes own (channel, 32 or 16 tokens): chunk cumsum, decay factors, scaled operands
//              written once to LDS (2 exps per element)
//   A/P        20 MFMA tiles (10 per matrix) shared by the waves (16x16x32, fp32 accumulate)
//   T_bb       one wave inverts the four 16x16 unit-lower diagonal blocks of I + A (substitution)
//   state      per wave: Y = Kt S, O = Qt S (16x16x32), W by blocked forward substitution
//              (16x16x16), O += P W, S <- e^{G_n} S + Kb^T W; o stored straight from registers.
// Precision: products whose operands are range-bounded use fp16 (11-bit significand) in one
// pass; the diagonal A/P tiles (factors up to e^80), the triangular solve and P W use split bf16
// (hi*hi + hi*lo + lo*hi).  For fp32 inputs every product is split bf16.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;      // tokens per chunk
constexpr int BV = 64;      // state columns per workgroup (16 per wave)
constexpr int NTHR = 256;
constexpr int LA = CH + 4;  // padded row length of the 64x64 A / P tiles (floats)

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- MFMA wrappers --------------------------------------------------------------------------
// 16x16x32: lane (m, q) = (lane % 16, lane / 16) supplies row m of A (column m of B) and eight
// K-slots.  Throughout this file K-slot i of lane group q stands for K index
//     i < 4 :  4q + i          i >= 4 :  16 + 4q + (i - 4)
// (applied identically to both operands), so the two 16-row output tiles of an earlier MFMA,
// whose lane (n, q) holds rows 4q..4q+3 each, form a B operand without any shuffle.
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 h = static_cast<__bf16>(x[i]);
        hi[i] = h;
        lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(h));
    }
}

__device__ __forceinline__ f32x4 mma32_x3(const float (&a)[8], const float (&b)[8], f32x4 acc) {
    bf16x8 ah, al, bh, bl;
    split_bf16(a, ah, al);
    split_bf16(b, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ f16x8 to_f16x8(const float (&x)[8]) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<_Float16>(x[i]);
    return r;
}

__device__ __forceinline__ f32x4 mma32_f16(const float (&a)[8], const float (&b)[8], f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(to_f16x8(a), to_f16x8(b), acc, 0, 0, 0);
}

template <bool X3>
__device__ __forceinline__ f32x4 mma32(const float (&a)[8], const float (&b)[8], f32x4 acc) {
    if constexpr (X3) return mma32_x3(a, b, acc);
    else return mma32_f16(a, b, acc);
}

// 16x16x16 (bf16, split): lane (m, q) holds K indices 4q..4q+3; the output layout equals the
// B-operand layout, so a result feeds the next product directly.
__device__ __forceinline__ void split_bf16_4(const float (&x)[4], s16x4& hi, s16x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 h = static_cast<__bf16>(x[i]);
        const __bf16 l = static_cast<__bf16>(x[i] - static_cast<float>(h));
        hi[i] = __builtin_bit_cast(short, h);
        lo[i] = __builtin_bit_cast(short, l);
    }
}

__device__ __forceinline__ f32x4 mma16_x3(const float (&a)[4], const float (&b)[4], f32x4 acc) {
    s16x4 ah, al, bh, bl;
    split_bf16_4(a, ah, al);
    split_bf16_4(b, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    return acc;
}

// Prefetched raw inputs of one staging lane: fp32 as is, bf16 packed two per register.
template <int DT, int N>
struct RawVec;
template <int N>
struct RawVec<KDA_F32, N> {
    float v[N];
    __device__ __forceinline__ void load(const void* p, int i, int64_t e, bool ok) {
        v[i] = ok ? static_cast<const float*>(p)[e] : 0.f;
    }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <int N>
struct RawVec<KDA_BF16, N> {
    uint32_t v[(N + 1) / 2];
    __device__ __forceinline__ void load(const void* p, int i, int64_t e, bool ok) {
        const uint32_t b = ok ? static_cast<uint32_t>(static_cast<const uint16_t*>(p)[e]) : 0u;
        if (i & 1) v[i / 2] = (v[i / 2] & 0xffffu) | (b << 16);
        else v[i / 2] = b;
    }
    __device__ __forceinline__ float get(int i) const {
        return (i & 1) ? __uint_as_float(v[i / 2] & 0xffff0000u) : __uint_as_float(v[i / 2] << 16);
    }
};

__device__ __forceinline__ void ld4(const float* p, float* dst) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
}

// ---- the fused kernel -----------------------------------------------------------------------
template <int DK, int IDT, int GDT, int ODT, bool PRECISE>
__global__ void __launch_bounds__(NTHR, 1) chunk_fwd_kernel(ChunkArgs p, int32_t n_vblk) {
    constexpr int LDK = DK + 4;          // padded row length of the [64][DK] staging arrays
    constexpr int KSTEPS = DK / 32;      // 32-channel K-steps
    constexpr int CT = DK / 16;          // 16-channel tiles of the state
    constexpr int TPC = NTHR / DK;       // staging lanes per channel (2 or 4)
    constexpr int TPT = CH / TPC;        // tokens per staging lane (32 or 16)
    constexpr int BPT = TPT / 16;        // 16-token blocks per staging lane (2 or 1)
    constexpr int REG4 = (CH * LDK > 2 * CH * LA) ? CH * LDK : 2 * CH * LA;

    __shared__ __attribute__((aligned(16))) float sm[3 * CH * LDK + REG4];
    __shared__ __attribute__((aligned(16))) float sTbb[4][16][16];
    __shared__ float sRb[5][DK];         // R_0 .. R_3 (block references), G_63
    __shared__ float sE[4][DK];          // e^{R_b}
    __shared__ float sF[3][DK];          // e^{R_b - R_{j+1}} for (b, j) = (2,0), (3,0), (3,1)
    __shared__ float sH[4][DK];          // e^{G_63 - R_{j+1}}
    __shared__ float sGam[DK];           // e^{G_63}
    __shared__ float sSeg[TPC][DK];      // per-segment g totals
    __shared__ float sBeta[CH];

    float* const sKR = sm;                    // k_r e^{G_r - R_b}
    float* const sQR = sm + CH * LDK;         // q_r e^{G_r - R_b}
    float* const sKB = sm + 2 * CH * LDK;     // k_s e^{R_{j+1} - G_s}
    float* const sKD = sm + 3 * CH * LDK;     // k_s e^{R_j - G_s}   (A/P phase only)
    float* const sA = sm + 3 * CH * LDK;      // beta-scaled strict-lower A (after the A/P phase)
    float* const sP = sA + CH * LA;           // lower P

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lq = lane >> 4;

    // Workgroup -> (unit, column block).  The column blocks of one unit are placed 8 workgroup
    // ids apart so they land on the same XCD and share its L2 for the unit's q/k/g reads.
    const int64_t units = static_cast<int64_t>(p.n_seqs) * p.H;
    const int64_t bid = blockIdx.x;
    const int64_t grp = bid / (8 * n_vblk), rem = bid % (8 * n_vblk);
    const int vb = static_cast<int>(rem / 8);
    const int64_t unit = grp * 8 + rem % 8;
    if (unit >= units) return;
    const int n = static_cast<int>(unit / p.H), h = static_cast<int>(unit % p.H);
    const int DV = p.dv;
    const int n0 = vb * BV + wave * 16;        // this wave's first state column

    int64_t bos, len;
    if (p.cu) {
        bos = p.cu[n];
        len = static_cast<int64_t>(p.cu[n + 1]) - bos;
    } else {
        bos = static_cast<int64_t>(n) * p.T;
        len = p.T;
    }
    const int64_t H = p.H;

    // ---- state tiles: lane (ln, lq) of tile i holds S[16i + 4lq + r][n0 + ln]
    f32x4 S[CT];
    const int64_t sbase = unit * DK * DV;
#pragma unroll
    for (int i = 0; i < CT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = p.h0 ? p.h0[sbase + static_cast<int64_t>(16 * i + 4 * lq + r) * DV + n0 + ln] : 0.f;
    }

    // staging lane identity
    const int sc = tid % DK;          // channel
    const int seg = tid / DK;         // token segment [seg*TPT, seg*TPT + TPT)

    RawVec<GDT, TPT> pg;              // prefetched raw inputs of the next chunk
    RawVec<IDT, TPT> pk, pq;
    auto prefetch = [&](int64_t t0, int nt) {
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int r = seg * TPT + i;
            const bool ok = r < nt;
            const int64_t e = ok ? ((bos + t0 + r) * H + h) * DK + sc : 0;
            pg.load(p.g, i, e, ok);
            pk.load(p.k, i, e, ok);
            pq.load(p.q, i, e, ok);
        }
    };

    const int64_t nchunks = (len + CH - 1) / CH;
    if (nchunks > 0) prefetch(0, static_cast<int>(len < CH ? len : CH));

    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t t0 = ci * CH;
        const int nt = static_cast<int>((len - t0) < CH ? (len - t0) : CH);

        // ---------------- staging 1: chunk cumsum per (channel, segment)
        float G[TPT];
        {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < TPT; ++i) { run += pg.get(i); G[i] = run; }
            sSeg[seg][sc] = run;
        }
        if (tid < CH) sBeta[tid] = (tid < nt) ? load_as_f32<IDT>(p.beta, (bos + t0 + tid) * H + h) : 0.f;
        // this wave's V values for the state phase: V[16b + 4lq + r][n0 + ln]
        float vpre[16];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * b + 4 * lq + r;
                vpre[4 * b + r] = (row < nt)
                    ? load_as_f32<IDT>(p.v, ((bos + t0 + row) * H + h) * DV + n0 + ln) : 0.f;
            }
        __syncthreads();

        // ---------------- staging 2: chunk-global prefix, block references
        {
            float base = 0.f, total = 0.f;
#pragma unroll
            for (int s = 0; s < TPC; ++s) {
                const float x = sSeg[s][sc];
                if (s < seg) base += x;
                total += x;
            }
#pragma unroll
            for (int i = 0; i < TPT; ++i) G[i] += base;
            // R_{j+1} = G at the last token of block j
#pragma unroll
            for (int bl = 0; bl < BPT; ++bl) sRb[seg * BPT + bl + 1][sc] = G[16 * bl + 15];
            if (seg == 0) sRb[0][sc] = 0.f;
            // sRb[4] (= G_63) is written by the last segment above
            (void)total;
        }
        // next chunk's raw inputs: issue now, consumed at the next iteration
        const RawVec<IDT, TPT> kcur = pk, qcur = pq;
        if (ci + 1 < nchunks) {
            const int64_t t1 = t0 + CH;
            prefetch(t1, static_cast<int>((len - t1) < CH ? (len - t1) : CH));
        }
        __syncthreads();

        // ---------------- staging 3: scaled operands (2 exps per element) and small factors
#pragma unroll
        for (int bl = 0; bl < BPT; ++bl) {
            const int j = seg * BPT + bl;                 // block index of these 16 tokens
            const float Rj = sRb[j][sc];
            const float Ge = sRb[j + 1][sc];
            const float invD = __expf(Rj - Ge);           // e^{R_j - G_{e_j}} in [1, e^80]
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int ti = 16 * bl + i;
                const int r = 16 * j + i;
                const float gr = G[ti];
                const float er = __expf(gr - Rj);         // <= 1
                const float eb = __expf(Ge - gr);         // <= 1
                const float kv = kcur.get(ti);
                const float kb = kv * eb;
                sKR[r * LDK + sc] = kv * er;
                sQR[r * LDK + sc] = qcur.get(ti) * er;
                sKB[r * LDK + sc] = kb;
                sKD[r * LDK + sc] = kb * invD;
            }
        }
        if (tid < DK) {
            const int c = tid;
            const float R0 = 0.f, R1 = sRb[1][c], R2 = sRb[2][c], R3 = sRb[3][c], G63 = sRb[4][c];
            sE[0][c] = 1.f;
            sE[1][c] = __expf(R1);
            sE[2][c] = __expf(R2);
            sE[3][c] = __expf(R3);
            sF[0][c] = __expf(R2 - R1);   // (b, j) = (2, 0)
            sF[1][c] = __expf(R3 - R1);   // (3, 0)
            sF[2][c] = __expf(R3 - R2);   // (3, 1)
            sH[0][c] = __expf(G63 - R1);
            sH[1][c] = __expf(G63 - R2);
            sH[2][c] = __expf(G63 - R3);
            sH[3][c] = 1.f;
            sGam[c] = __expf(G63 - R0);
        }
        __syncthreads();

        // ---------------- A / P tiles.  Diagonal tiles first: they are the only readers of sKD,
        // which A and P overwrite.  Wave w owns the diagonal tiles (mat, b) = (w & 1, w >> 1) and
        // (w & 1, (w >> 1) + 2), then the off-diagonal tiles w, w + 4, w + 8 of the twelve.
        auto ap_tile = [&](int mat, int b, int j) -> f32x4 {
            const float* rowp = (mat ? sQR : sKR) + (16 * b + ln) * LDK;
            const float* colp = (j == b ? sKD : sKB) + (16 * j + ln) * LDK;
            const float* fp = (j + 1 < b) ? sF[(b == 2) ? 0 : (j == 0 ? 1 : 2)] : nullptr;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int c0 = 32 * kk + 4 * lq, c1 = c0 + 16;
                float a[8], bb[8];
                ld4(rowp + c0, a);
                ld4(rowp + c1, a + 4);
                if (fp) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) { a[i] *= fp[c0 + i]; a[4 + i] *= fp[c1 + i]; }
                }
                ld4(colp + c0, bb);
                ld4(colp + c1, bb + 4);
                if (PRECISE || j == b) acc = mma32_x3(a, bb, acc);
                else acc = mma32_f16(a, bb, acc);
            }
            return acc;
        };
        auto ap_store = [&](int mat, int b, int j, const f32x4& acc) {
            float* dst = mat ? sP : sA;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * b + 4 * lq + r;      // token r of the chunk
                const int col = 16 * j + ln;              // token s
                float x = acc[r];
                if (mat == 0) x = (col < row) ? x * sBeta[row] : 0.f;
                else x = (col <= row) ? x : 0.f;
                dst[row * LA + col] = x;
            }
        };
        const int dmat = wave & 1, db0 = wave >> 1;
        const f32x4 dacc0 = ap_tile(dmat, db0, db0);
        const f32x4 dacc1 = ap_tile(dmat, db0 + 2, db0 + 2);
        __syncthreads();   // everyone is done with sKD: A and P may overwrite it
        ap_store(dmat, db0, db0, dacc0);
        ap_store(dmat, db0 + 2, db0 + 2, dacc1);
#pragma unroll 1
        for (int t = wave; t < 12; t += 4) {
            const int mat = t & 1, pr = t >> 1;        // pr -> (b, j): (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
            const int b = pr < 1 ? 1 : pr < 3 ? 2 : 3;
            const int j = pr - (b * (b - 1)) / 2;
            ap_store(mat, b, j, ap_tile(mat, b, j));
        }
        // P tiles above the diagonal that the 32-token K-steps of P W read: (0,1) and (2,3)
        if (wave == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sP[(4 * lq + r) * LA + 16 + ln] = 0.f;
                sP[(32 + 4 * lq + r) * LA + 48 + ln] = 0.f;
            }
        }
        __syncthreads();

        // ---------------- T_bb = (I + A_bb)^{-1} (wave 0) ; Y = Kt S and O = Qt S (all waves)
        if (wave == 0) {
            const int b = lq, jc = ln;                     // block, column of T_bb
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == jc) ? 1.f : 0.f;
                const float* arow = sA + (16 * b + r) * LA + 16 * b;
#pragma unroll
                for (int sp = 0; sp < r; ++sp) s -= arow[sp] * t[sp];
                t[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sTbb[b][r][jc] = t[r];
        }

        // S as the B operand of 32-channel K-steps: c-tiles 2kk and 2kk+1
        f32x4 Y[4], O[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) { Y[b] = zero4(); O[b] = zero4(); }
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            float sb[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) { sb[r] = S[2 * kk][r]; sb[4 + r] = S[2 * kk + 1][r]; }
            const int c0 = 32 * kk + 4 * lq, c1 = c0 + 16;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float ak[8], aq[8];
                ld4(sKR + (16 * b + ln) * LDK + c0, ak);
                ld4(sKR + (16 * b + ln) * LDK + c1, ak + 4);
                ld4(sQR + (16 * b + ln) * LDK + c0, aq);
                ld4(sQR + (16 * b + ln) * LDK + c1, aq + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e0 = sE[b][c0 + i], e1 = sE[b][c1 + i];
                    ak[i] *= e0; ak[4 + i] *= e1;
                    aq[i] *= e0; aq[4 + i] *= e1;
                }
                Y[b] = mma32<PRECISE>(ak, sb, Y[b]);
                O[b] = mma32<PRECISE>(aq, sb, O[b]);
            }
        }
        __syncthreads();   // sTbb ready

        // ---------------- W by blocked forward substitution (per wave, its 16 columns)
        f32x4 W[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4 R;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * b + 4 * lq + r;
                R[r] = sBeta[row] * (vpre[4 * b + r] - Y[b][r]);
            }
#pragma unroll
            for (int j = 0; j < b; ++j) {
                float a4[4], w4[4];
                ld4(sA + (16 * b + ln) * LA + 16 * j + 4 * lq, a4);
#pragma unroll
                for (int i = 0; i < 4; ++i) { a4[i] = -a4[i]; w4[i] = W[j][i]; }
                R = mma16_x3(a4, w4, R);
            }
            float t4[4], r4[4];
            ld4(&sTbb[b][ln][4 * lq], t4);
#pragma unroll
            for (int i = 0; i < 4; ++i) r4[i] = R[i];
            W[b] = mma16_x3(t4, r4, zero4());
        }

        // ---------------- O += P W, store o
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int kk = 0; kk <= b / 2; ++kk) {
                float pa[8], wb[8];
                ld4(sP + (16 * b + ln) * LA + 32 * kk + 4 * lq, pa);
                ld4(sP + (16 * b + ln) * LA + 32 * kk + 16 + 4 * lq, pa + 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) { wb[r] = W[2 * kk][r]; wb[4 + r] = W[2 * kk + 1][r]; }
                O[b] = mma32_x3(pa, wb, O[b]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * b + 4 * lq + r;
                if (row < nt)
                    store_from_f32<ODT>(p.o, ((bos + t0 + row) * H + h) * DV + n0 + ln, p.scale * O[b][r]);
            }
        }

        // ---------------- S <- e^{G_n} S + Kb^T W
#pragma unroll
        for (int i = 0; i < CT; ++i) {
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = S[i][r] * sGam[16 * i + 4 * lq + r];
            const int c = 16 * i + ln;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float ka[8], wb[8];
                const float h0 = sH[2 * kk][c], h1 = sH[2 * kk + 1][c];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ka[r] = sKB[(32 * kk + 4 * lq + r) * LDK + c] * h0;
                    ka[4 + r] = sKB[(32 * kk + 16 + 4 * lq + r) * LDK + c] * h1;
                    wb[r] = W[2 * kk][r];
                    wb[4 + r] = W[2 * kk + 1][r];
                }
                acc = mma32<PRECISE>(ka, wb, acc);
            }
            S[i] = acc;
        }
        __syncthreads();   // LDS is rewritten by the next chunk's staging
    }

    if (p.hT) {
#pragma unroll
        for (int i = 0; i < CT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.hT[sbase + static_cast<int64_t>(16 * i + 4 * lq + r) * DV + n0 + ln] = S[i][r];
    }
}

template <int DK, int IDT, int GDT, int ODT>
hipError_t launch_t(const ChunkArgs& a, hipStream_t stream) {
    const int32_t n_vblk = a.dv / BV;
    const int64_t units = static_cast<int64_t>(a.n_seqs) * a.H;
    const int64_t groups = (units + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups * 8 * n_vblk));
    if (IDT == KDA_F32)
        hipLaunchKernelGGL((chunk_fwd_kernel<DK, IDT, GDT, ODT, true>), grid, dim3(NTHR), 0, stream, a, n_vblk);
    else
        hipLaunchKernelGGL((chunk_fwd_kernel<DK, IDT, GDT, ODT, false>), grid, dim3(NTHR), 0, stream, a, n_vblk);
    return hipGetLastError();
}

template <int DK>
hipError_t dispatch(const ChunkArgs& a, hipStream_t s) {
#define KDA_CH(I, G, O) \
    if (a.in_dtype == I && a.g_dtype == G && a.o_dtype == O) return launch_t<DK, I, G, O>(a, s);
    KDA_CH(KDA_BF16, KDA_F32, KDA_BF16)
    KDA_CH(KDA_BF16, KDA_F32, KDA_F32)
    KDA_CH(KDA_BF16, KDA_BF16, KDA_BF16)
    KDA_CH(KDA_BF16, KDA_BF16, KDA_F32)
    KDA_CH(KDA_F32, KDA_F32, KDA_F32)
    KDA_CH(KDA_F32, KDA_F32, KDA_BF16)
    KDA_CH(KDA_F32, KDA_BF16, KDA_F32)
    KDA_CH(KDA_F32, KDA_BF16, KDA_BF16)
#undef KDA_CH
    return hipErrorInvalidValue;
}

}  // namespace

size_t chunk_workspace_bytes(int32_t, int64_t, int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream) {
    if (a.dk == 128) return dispatch<128>(a, stream);
    return dispatch<64>(a, stream);
}

}  // namespace kda
