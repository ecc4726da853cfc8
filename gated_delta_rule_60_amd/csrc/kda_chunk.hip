// kda_chunk.hip -- chunked KDA prefill on gfx950: an intra-block kernel and a state-passing kernel.
//
// Pages (titles as published):
//   [bagrov] "Архитектура Kimi K3: как открытая модель с миллионным контекстом конкурирует с
//            лидерами рынка" (bagrov.by): § "Как архитектура Kimi K3 удерживает миллион токенов
//            контекста" (fixed state, delta rule, bounded forget factor), § "Уровень чипа:
//            специализированное ядро FlashKDA" (two steps: the tokens of a block are processed
//            fully in parallel, then the state is passed on, spread over independent heads).
//   [habr]   "Как устроена Kimi K3: …" (savepearlharbor.com), § "Последовательность: три KDA на
//            один глобальный MLA" (g = g_min*sigmoid(exp(A) z) with g_min = -5 keeps the running
//            decay inside the bf16 range, so every causal 16-token block, diagonal ones included,
//            is a dense matrix product).
//
// Block form (derived from the token recurrence).  For a block of n <= 16 tokens entering with
// state S, G_r = sum_{t<=r} g_t (per key channel, restarting at the block), G_15 its end value:
//   Kt = e^G * K,  Qt = e^G * Q,  Kb = e^{G_15 - G} * K,  Kd = e^{-G} * K     (elementwise)
//   A = beta * strict_lower(Kt Kd^T),  P = lower(Qt Kd^T)                  (16 x 16)
//   T' = (I + A)^{-1} Diag(beta)                                            (UT transform)
//   W  = T' (V - Kt S)        row r of W is beta_r times token r's delta-rule innovation
//   O  = scale * (Qt S + P W),          S <- Diag(e^{G_15}) S + Kb^T W
// Kt, Qt, Kb lie in [-1, 1] (factors <= 1); Kd's factor is at most e^{16*5} = e^80, inside the
// bf16 / fp32 range (e^88.7): the bound on g is what makes the diagonal block a plain dense
// product.  For 16-bit inputs one state step covers two such blocks (32 tokens): the same form
// with G taken from the first block's start, its 32 x 32 A and P assembled from 16 x 16 tiles
// whose exponents stay within e^{+-80} (the cross tiles use factors <= 1 referenced at the
// blocks' boundary), and T' block-triangular.  Successive steps are chained through S, so a
// 64-token chunk's triangular system is solved blockwise, the coupling going through the state.
//
// 1. Intra-block kernel (everything that does not depend on S; fully parallel): writes one
//    record per (head, record slot) to the workspace -- -Kt, Qt, Kb^T in their MFMA formats,
//    the diagonal blocks of T', the cross tile -C, P, the step's e^{G_last} - 1.
//    16-bit inputs (chunk_intra_tok_kernel): one wave per (32-token record, head); each lane
//    owns one token of each 16-token sub-block and the channels of its record unit; inputs
//    arrive by direct-to-LDS loads, the cumsums are DPP scans across the lanes, A and P are fp32
//    MFMAs fed from registers, the diagonal blocks of T' come by substitution; the off-diagonal
//    block T'_10 = -T'_11 C T'_00 is left to the state pass, which applies it as two products.
//    fp32 inputs (chunk_intra_kernel, split-bf16 records of 16 tokens): each lane owns 4 tokens
//    x 4 channels; quad-lane cumsum, A and P on MFMA from split-bf16 operands staged in LDS.
// 2. State-passing kernel (the sequential part): one workgroup of STATE_WAVES computing waves
//    per (sequence, head, 16 STATE_WAVES state columns); each wave owns 16 state columns in fp32
//    accumulators for the whole sequence.  A chunk's two records and its V rows stream into
//    double-buffered LDS while the previous chunk is processed; in the two-wave workgroups two
//    more waves issue those transfers and store o from an LDS stage, so the computing waves
//    issue no memory instructions in the loop.  Optionally it stores the state every k tokens
//    (checkpoints).  Long sequences with few (sequence, head) units run as
//    segments: pass 1 (the segments' affine pairs; chunk_pair_kernel at d_k = d_v = 128), a scan
//    of the pairs, pass 2 (see the segment section below).
// Launches with 16-bit inputs at d_k = d_v = 128 and at least 256 (sequence, head) units run the
// single fused kernel of kda_fused.hip instead, with no workspace.
// Precision (16-bit inputs): A and P of each 16-token block are fp32 products; every operand of
// the state pass is range-bounded and runs in fp16 (11-bit significand) with fp32 accumulation.
// For fp32 inputs every product is split bf16 (hi*hi + hi*lo + lo*hi).
#include <mutex>
#include <type_traits>

#include "kda_chunk_util.hpp"

namespace kda {
namespace {

constexpr int BLK = 16;     // tokens per block (one state step)
// Waves per state-kernel workgroup, 16 state columns each: 2 in the whole-sequence pass (more
// CUs, each streaming the records once per 32 columns, measured faster than 4), 4 in the segment
// passes (8 when d_k = d_v = 128).
constexpr int STATE_WAVES = 2;
constexpr int SEG_WAVES = 4;
constexpr int STATE_SLICES = 1;  // transfer slices of a chunk in the state pass without helpers
// Helper waves of the state pass: a workgroup of at most two computing waves uses at most two of
// a CU's four SIMDs, so as many more waves only issue its transfers (the computing waves then
// never stall on a run of memory instructions).
constexpr int state_helpers(int nw) { return nw <= 2 ? nw : 0; }

// ---- MFMA wrappers (operands already in their 16-bit format) --------------------------------
__device__ __forceinline__ f32x4 mfma32_bf16_x3(const bf16x8& ah, const bf16x8& al,
                                                const bf16x8& bh, const bf16x8& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16_x3(const s16x4& ah, const s16x4& al,
                                                const s16x4& bh, const s16x4& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
}

// ---- quad-lane moves (lanes 4k..4k+3) -------------------------------------------------------
// DPP quad_perm: lane 4k+i receives the value of lane 4k+perm[i].
template <int PERM>
__device__ __forceinline__ float quad_perm(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), PERM, 0xf, 0xf, false));
}
constexpr int QP_PREV1 = 0 | (0 << 2) | (1 << 4) | (2 << 6);   // [0,0,1,2]
constexpr int QP_PREV2 = 0 | (0 << 2) | (0 << 4) | (1 << 6);   // [0,0,0,1]
constexpr int QP_LAST = 3 | (3 << 2) | (3 << 4) | (3 << 6);    // [3,3,3,3]

// Record of one (head, block slot) in the workspace (byte offsets).  E = 16 * DK elements per
// array.  A fast record covers 32 tokens: two 16-token sub-blocks, one 32-token state step; a
// precise record covers one 16-token block.
//   fast   : first what every state pass reads -- [-Kt_0 frag32][Kb^T][-Kt_1 frag32][Kb^T] (fp16
//            [16][DK] arrays; the two Kb^T arrays hold Kb^T of both sub-blocks in fragKb order,
//            tiles 0 .. DK/32 - 1 in the first, the rest in the second), T'_00, -C, T'_11 (fp16
//            fragT) and e^{G_31} - 1 (DK fp32), HEAD bytes, a whole number of 1 KB units at
//            d_k = 128 -- then what only output passes read: [Qt_0 frag32][Qt_1 frag32] and
//            P_00, P_10, P_11 (fp16 fragT, [row sub-block][column sub-block]).  Kt, Qt are scaled
//            from the record's first token, Kb from its last, so every exponent is <= 0.  Kt is
//            stored negated so that the state passes form V - Kt S as one product accumulated
//            onto V.
//   precise: [Kt hi][Kt lo][Qt hi][Qt lo] (bf16 frag32) [Kb^T hi][Kb^T lo] (bf16 frag16), then T'
//            and P (bf16 hi, lo; fragT), then e^{G_15} - 1 (DK fp32).
//   Qt and P carry the output scale.  |P| <= |q| |k| <= 1 for L2-normalised q, k, inside fp16.
// An all-zero record is the identity step (W = 0, S unchanged), which lets the state pass run
// every chunk as two records without branches: records past a sequence's end read zeros.
template <int DK, bool PRECISE>
struct Rec {
    static constexpr int TOK = PRECISE ? 16 : 32;       // tokens per record
    static constexpr int E = BLK * DK;
    static constexpr int NA = 6;                        // 16-bit [16][DK] arrays
    static constexpr int E2 = 2 * E;                    // bytes of one of them
    static constexpr int TB = PRECISE ? 1024 : 1536;    // the T' tiles, and the P tiles
    // fast layout (the precise one: arrays 0..5, T', P, decay)
    static constexpr int OFF_KB_LO = E2, OFF_KT1 = 2 * E2, OFF_KB_HI = 3 * E2;
    static constexpr int OFF_T = PRECISE ? NA * E2 : 4 * E2;
    static constexpr int OFF_G = PRECISE ? OFF_T + 2 * TB : OFF_T + TB;
    static constexpr int HEAD = OFF_G + DK * 4;         // fast: the part every state pass reads
    static constexpr int OFF_QT0 = HEAD, OFF_QT1 = HEAD + E2;
    static constexpr int OFF_P = PRECISE ? OFF_T + TB : HEAD + 2 * E2;
    static constexpr int BYTES = PRECISE ? HEAD : OFF_P + TB;
    static_assert(BYTES % 16 == 0 && HEAD % 16 == 0, "record alignment");
    // fast: the byte offset of the state pass's A operand a (-Kt_0, Qt_0, -Kt_1, Qt_1)
    static constexpr int fa_off(int a) { return a == 0 ? 0 : a == 1 ? OFF_QT0 : a == 2 ? OFF_KT1 : OFF_QT1; }
    // fast: Kb^T tile i
    static constexpr int kb_off(int i) { return kb_tile_off(i, DK / 16, OFF_KB_LO, OFF_KB_HI); }
};

// Raw inputs held by one staging lane: 4 tokens x CPT channels; bf16 packed two per register.
template <int DT, int N>
struct Raw;
template <int N>
struct Raw<KDA_F32, N> {
    float v[N];
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <int N>
struct Raw<KDA_BF16, N> {
    uint32_t v[N / 2];
    __device__ __forceinline__ float get(int i) const {
        return (i & 1) ? __uint_as_float(v[i / 2] & 0xffff0000u) : __uint_as_float(v[i / 2] << 16);
    }
};
// Inputs are read exactly once: non-temporal loads keep them out of the caches, which are
// better spent on the workspace records that the state pass reads back.
typedef unsigned int u32x4nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2nt __attribute__((ext_vector_type(2)));
template <int DT, int CPT, int N>
__device__ __forceinline__ void load_row(Raw<DT, N>& dst, int slot, const void* base, int32_t e,
                                         bool ok) {
    if constexpr (DT == KDA_F32) {
        const float* src = static_cast<const float*>(base) + e;
#pragma unroll
        for (int u = 0; u < CPT / 4; ++u) {
            u32x4nt x = {0u, 0u, 0u, 0u};
            if (ok) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4nt*>(src + 4 * u));
            dst.v[slot * CPT + 4 * u + 0] = __uint_as_float(x[0]);
            dst.v[slot * CPT + 4 * u + 1] = __uint_as_float(x[1]);
            dst.v[slot * CPT + 4 * u + 2] = __uint_as_float(x[2]);
            dst.v[slot * CPT + 4 * u + 3] = __uint_as_float(x[3]);
        }
    } else {
        const uint16_t* src = static_cast<const uint16_t*>(base) + e;
        if constexpr (CPT == 8) {
            u32x4nt x = {0u, 0u, 0u, 0u};
            if (ok) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4nt*>(src));
            dst.v[slot * 4 + 0] = x[0]; dst.v[slot * 4 + 1] = x[1];
            dst.v[slot * 4 + 2] = x[2]; dst.v[slot * 4 + 3] = x[3];
        } else {
            u32x2nt x = {0u, 0u};
            if (ok) x = __builtin_nontemporal_load(reinterpret_cast<const u32x2nt*>(src));
            dst.v[slot * 2 + 0] = x[0]; dst.v[slot * 2 + 1] = x[1];
        }
    }
}

template <int NP>
__device__ __forceinline__ void store_words(void* dst, const uint32_t (&w)[NP]) {
    if constexpr (NP == 4) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
}

// Locate the record slot of a workgroup: sequence n, record j inside it (TOK tokens each), or
// false when the slot is past its sequence's end.  Slot bases: n * ceil(T/TOK) for fixed-length
// batches, floor(bos_n/TOK) + n for packed ones (ceil(len/TOK) <= floor(len/TOK) + 1 keeps them
// disjoint, and floor(bos/TOK) + ceil(len/TOK) <= ceil(T/TOK) keeps them below the
// T/TOK + N + 1 slots of the workspace).
template <int TOK>
__device__ __forceinline__ bool locate_slot(const ChunkArgs& p, int64_t slot, int& n,
                                            int64_t& j, int64_t& bos, int64_t& len) {
    if (p.cu) {
        int lo = 0, hi = p.n_seqs - 1;
        while (lo < hi) {                 // largest n with base(n) <= slot
            const int mid = (lo + hi + 1) >> 1;
            const int64_t base = seq_start(p, mid) / TOK + mid;
            if (base <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        int64_t end;
        seq_bounds(p, n, bos, end);
        len = end - bos;
        j = slot - (bos / TOK + n);
    } else {
        const int64_t nrec = (p.T + TOK - 1) / TOK;
        if (nrec == 0) return false;
        n = static_cast<int>(slot / nrec);
        j = slot % nrec;
        if (n >= p.n_seqs) return false;
        bos = static_cast<int64_t>(n) * p.T;
        len = p.T;
    }
    return j >= 0 && TOK * j < len;
}

// ============================================================================================
// 1. intra-block kernel for fp32 inputs (split-bf16 records): one wave per (block slot, head)
// ============================================================================================
template <int DK, int IDT, int GDT, bool PRECISE, bool GATE>
__global__ void __launch_bounds__(64) chunk_intra_kernel(ChunkArgs p, int64_t nslots, uint8_t* ws) {
    static_assert(PRECISE, "16-bit inputs use chunk_intra_tok_kernel");
    using R = Rec<DK, PRECISE>;
    constexpr int PH = DK / 64;           // the channels are processed in phases of 64
    constexpr int LE = BLK * 64;          // elements of one [16][64] LDS operand array
    constexpr float LOG2E = 1.4426950408889634f;

    // split operands of one phase (reused by the next): 12 KB, so that 12 waves fit a CU.  Once
    // a phase's products are formed the same 12 KB stage its share of the record, which then
    // goes out in whole 1 KB wave stores (the record's fragment order scatters a lane's values).
    __shared__ __attribute__((aligned(16))) uint16_t sOps[6 * LE];
    uint16_t* const sKh = sOps;              // Kt hi / lo
    uint16_t* const sKl = sOps + LE;
    uint16_t* const sQh = sOps + 2 * LE;     // Qt hi / lo
    uint16_t* const sQl = sOps + 3 * LE;
    uint16_t* const sDh = sOps + 4 * LE;     // Kd hi / lo
    uint16_t* const sDl = sOps + 5 * LE;
    uint8_t* const stg = reinterpret_cast<uint8_t*>(sOps);
    constexpr int WIN = 2 * BLK * 64;        // bytes of one record array's share of a phase
    __shared__ __attribute__((aligned(16))) float sA[16][16];
    __shared__ float sBeta[16];

    const int lane = threadIdx.x;
    const int ln = lane & 15, lq = lane >> 4;
    const int cg = lane >> 2, sub = lane & 3;

    const int64_t H = p.H;
    const int64_t gu = global_unit(p, blockIdx.x);
    const int64_t slot = gu / H;
    const int h = static_cast<int>(gu % H);
    int n;
    int64_t j, bos, len;
    if (!locate_slot<BLK>(p, slot, n, j, bos, len)) return;
    const int64_t t0 = BLK * j;
    const int nt = static_cast<int>((len - t0) < BLK ? (len - t0) : BLK);
    uint8_t* rec = ws + (static_cast<int64_t>(h) * nslots + slot) * R::BYTES;

    // ---- inputs of every phase, loaded up front: in phase ph, lane (cg, sub) holds rows
    // 4sub .. 4sub+3, channels 64ph + 4cg .. +3; beta goes to LDS from lanes 0..15
    Raw<GDT, 16> pg[PH];                  // g, or z when the gate is fused
    Raw<IDT, 16> pk[PH], pq[PH];
    {
        const int64_t row0 = (bos + t0) * H + h;
        const int32_t kstride = static_cast<int32_t>(H) * DK;
        const void* gbase = static_cast<const char*>(p.g) + row0 * DK * (GDT == KDA_F32 ? 4 : 2);
        const void* kbase = static_cast<const char*>(p.k) + row0 * DK * (IDT == KDA_F32 ? 4 : 2);
        const void* qbase = static_cast<const char*>(p.q) + row0 * DK * (IDT == KDA_F32 ? 4 : 2);
#pragma unroll
        for (int ph = 0; ph < PH; ++ph)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * sub + i;
                const bool ok = r < nt;
                const int32_t e = ok ? r * kstride + 64 * ph + 4 * cg : 0;
                load_row<GDT, 4>(pg[ph], i, gbase, e, ok);
                load_row<IDT, 4>(pk[ph], i, kbase, e, ok);
                load_row<IDT, 4>(pq[ph], i, qbase, e, ok);
            }
        if (lane < 16) {
            const void* bbase = static_cast<const char*>(p.beta) + row0 * (IDT == KDA_F32 ? 4 : 2);
            sBeta[lane] = (lane < nt) ? load_as_f32<IDT>(bbase, lane * static_cast<int32_t>(H)) : 0.f;
        }
    }

    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int ph = 0; ph < PH; ++ph) {
        const int c0 = 64 * ph + 4 * cg;                  // this lane's first channel
        if (ph > 0) __syncthreads();                      // the previous phase's reads are done

        // ---- fused gate: g = g_min * sigmoid(exp(A) z) from z, the same arithmetic as kda_gate;
        // rows past the block's tokens get g = 0 like the zero-filled g of the unfused path
        GateRate ea[4];
        if constexpr (GATE) {
            const float* a = p.gate_A + static_cast<int64_t>(h) * DK + c0;
#pragma unroll
            for (int c = 0; c < 4; ++c) ea[c] = gate_rate(a[c]);
        }
        auto gval = [&](int i, int c) -> float {
            if constexpr (GATE) return (4 * sub + i < nt) ? gate_log_decay(ea[c], pg[ph].get(i * 4 + c), p.g_min) : 0.f;
            else return pg[ph].get(i * 4 + c);
        };

        // ---- block cumsum (log2 units): own 4 tokens, then a scan over the 4 lanes of the group
        float G2[16];
        float G15[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // one explicit rounding: the fused-gate and g-given variants must not differ in
                // whether the compiler contracts this into an fma
                run = fmaf(gval(i, c), LOG2E, run);
                G2[i * 4 + c] = run;
            }
            float incl = run;
            const float u1 = quad_perm<QP_PREV1>(incl);
            if (sub >= 1) incl += u1;
            const float u2 = quad_perm<QP_PREV2>(incl);
            if (sub >= 2) incl += u2;
            const float excl = incl - run;
#pragma unroll
            for (int i = 0; i < 4; ++i) G2[i * 4 + c] += excl;
            G15[c] = quad_perm<QP_LAST>(incl);
        }

        // ---- decay factors, operands
        float gam[4];                                     // e^{G15}
#pragma unroll
        for (int c = 0; c < 4; ++c) gam[c] = fexp2(G15[c]);
        float kb[16];
        uint2 rw[R::NA][4];                               // this lane's record words, by array
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * sub + i;
            float kt[4], qt[4], kd[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float g2 = G2[i * 4 + c];
                const float e1 = fexp2(g2);               // e^{G}  <= 1
                const float kv = pk[ph].get(i * 4 + c);
                kt[c] = kv * e1;
                qt[c] = pq[ph].get(i * 4 + c) * (e1 * p.scale);   // the output scale rides on Qt and P
                kd[c] = kv * fexp2(-g2);                  // e^{-G} <= e^80
                kb[i * 4 + c] = kd[c] * gam[c];           // e^{G15 - G} <= 1
            }
            uint32_t wKh[2], wKl[2], wQh[2], wQl[2], wDh[2], wDl[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                split_pair(kt[2 * u], kt[2 * u + 1], wKh[u], wKl[u]);
                split_pair(qt[2 * u], qt[2 * u + 1], wQh[u], wQl[u]);
                split_pair(kd[2 * u], kd[2 * u + 1], wDh[u], wDl[u]);
            }
            const int off = tok_major<64>(r, 4 * cg);
            store_words<2>(sKh + off, wKh); store_words<2>(sKl + off, wKl);
            store_words<2>(sQh + off, wQh); store_words<2>(sQl + off, wQl);
            store_words<2>(sDh + off, wDh); store_words<2>(sDl + off, wDl);
            // record words: the state pass's Kt, Qt operands (frag32: four channels = 8 bytes)
            if constexpr (!PRECISE) {
                rw[0][i] = make_uint2(f16_pair(kt[0], kt[1]), f16_pair(kt[2], kt[3]));
                rw[1][i] = make_uint2(f16_pair(qt[0], qt[1]), f16_pair(qt[2], qt[3]));
            } else {
                rw[0][i] = make_uint2(wKh[0], wKh[1]);
                rw[1][i] = make_uint2(wKl[0], wKl[1]);
                rw[2][i] = make_uint2(wQh[0], wQh[1]);
                rw[3][i] = make_uint2(wQl[0], wQl[1]);
            }
        }
        // record words: Kb^T (frag16: the lane's 4 tokens of each channel are contiguous)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (!PRECISE) {
                rw[2][c] = make_uint2(f16_pair(kb[0 + c], kb[4 + c]), f16_pair(kb[8 + c], kb[12 + c]));
            } else {
                uint32_t h0, l0, h1, l1;
                split_pair(kb[0 + c], kb[4 + c], h0, l0);
                split_pair(kb[8 + c], kb[12 + c], h1, l1);
                rw[4][c] = make_uint2(h0, h1);
                rw[5][c] = make_uint2(l0, l1);
            }
        }
        // record: e^{G_15} - 1 (same absolute precision as e^{G_15} in fp32)
        if (sub == 0) {
            float* gr = reinterpret_cast<float*>(rec + R::OFF_G) + c0;
#pragma unroll
            for (int c = 0; c < 4; ++c) gr[c] = gam[c] - 1.f;
        }

        __syncthreads();   // the operand arrays (and beta) are read across lanes below

        // ---- this phase's share of A and P (16 x 16, contraction over its 64 channels)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int off = tok_major<64>(ln, 32 * kk + 8 * lq);
            const bf16x8 kh = *reinterpret_cast<const bf16x8*>(sKh + off);
            const bf16x8 kl = *reinterpret_cast<const bf16x8*>(sKl + off);
            const bf16x8 qh = *reinterpret_cast<const bf16x8*>(sQh + off);
            const bf16x8 ql = *reinterpret_cast<const bf16x8*>(sQl + off);
            const bf16x8 dh = *reinterpret_cast<const bf16x8*>(sDh + off);
            const bf16x8 dl = *reinterpret_cast<const bf16x8*>(sDl + off);
            accA = mfma32_bf16_x3(kh, kl, dh, dl, accA);
            accP = mfma32_bf16_x3(qh, ql, dh, dl, accP);
        }

        // ---- this phase's share of the record: array a holds bytes [a * 2E + WIN * ph, + WIN)
        __syncthreads();   // the operand arrays have been read
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int so = 2 * frag32(4 * sub + i, c0) - WIN * ph;
#pragma unroll
            for (int a = 0; a < (PRECISE ? 4 : 2); ++a)
                *reinterpret_cast<uint2*>(stg + a * WIN + so) = rw[a][i];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int so = 2 * frag16(c0 + c, 4 * sub) - WIN * ph;
#pragma unroll
            for (int a = (PRECISE ? 4 : 2); a < R::NA; ++a)
                *reinterpret_cast<uint2*>(stg + a * WIN + so) = rw[a][c];
        }
        __syncthreads();
#pragma unroll
        for (int a = 0; a < R::NA; ++a)
#pragma unroll
            for (int u = 0; u < WIN / 1024; ++u)
                *reinterpret_cast<uint4*>(rec + a * 2 * R::E + WIN * ph + (64 * u + lane) * 16) =
                    *reinterpret_cast<const uint4_ma*>(stg + a * WIN + (64 * u + lane) * 16);
    }
    // T' and P are staged too, then written with e^{G_15} - 1 already in place: bytes
    // [OFF_T, OFF_G) of the record
    constexpr int TAIL = R::OFF_G - R::OFF_T;
    uint16_t* const tT = reinterpret_cast<uint16_t*>(stg);
    uint16_t* const tP = reinterpret_cast<uint16_t*>(stg + (R::OFF_P - R::OFF_T));
    __syncthreads();   // the last phase's record share has been copied out
    {
        // lane (ln, lq) holds rows 4lq + i of column ln
        uint16_t* Ph = tP;
        uint16_t* Pl = tP + 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lq + i, s = ln;
            sA[r][s] = (s < r) ? accA[i] * sBeta[r] : 0.f;
            const float pval = (s <= r) ? accP[i] : 0.f;
            const uint16_t ph = bf16_bits(pval);
            Ph[fragT(r, s)] = ph;
            Pl[fragT(r, s)] = bf16_bits(pval - bf16_val(ph));
        }
    }
    __syncthreads();   // sA rows are read by other lanes

    // ---- T' = (I + A)^{-1} Diag(beta): forward substitution, lane j = column j; rows are read
    // one ahead of use and each row's dot product runs as four independent partial sums
    if (lane < 16) {
        const int jc = lane;
        float t[16];
        float4 nxt[4], cur[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) nxt[u] = *reinterpret_cast<const float4_ma*>(&sA[1][4 * u]);
        t[0] = (jc == 0) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
#pragma unroll
            for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
            if (r + 1 < 16) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (4 * u < r + 1) nxt[u] = *reinterpret_cast<const float4_ma*>(&sA[r + 1][4 * u]);
            }
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < r; ++sp) {
                const float4& c4 = cur[sp >> 2];
                const float a = (sp & 3) == 0 ? c4.x : (sp & 3) == 1 ? c4.y : (sp & 3) == 2 ? c4.z : c4.w;
                part[sp & 3] += a * t[sp];
            }
            t[r] = ((r == jc) ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
        }
        const float bj = sBeta[jc];
        uint16_t* Th = tT;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = t[r] * bj;
            if constexpr (!PRECISE) {
                Th[fragT(r, jc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
            } else {
                const uint16_t th = bf16_bits(x);
                Th[fragT(r, jc)] = th;
                Th[256 + fragT(r, jc)] = bf16_bits(x - bf16_val(th));
            }
        }
    }
    __syncthreads();   // T' and P staged
    for (int j = lane; j < TAIL / 16; j += 64)
        *reinterpret_cast<uint4*>(rec + R::OFF_T + 16 * j) = *reinterpret_cast<const uint4_ma*>(stg + 16 * j);
}

// ============================================================================================
// 1b. intra-block kernel for 16-bit inputs: one wave per (32-token record slot, head)
// ============================================================================================
// A record covers two 16-token sub-blocks s = 0, 1.  Lane (m, q) owns token m of each sub-block
// and, in every 32-channel group kk, the eight channels 32 kk + 16 (j >> 2) + 4 q + (j & 3),
// j = 0..7 -- exactly the channels its 16-byte unit of a frag32 record array holds.  Therefore:
//   * each sub-block's cumsum runs across the 16 lanes of a row (DPP shifts); G_15 is lane 15's;
//   * A_ss = beta * strict_lower(Kt_s Kd_s^T) and P_ss = lower(Qt_s Kd_s^T) are fp32 MFMAs
//     (16x16x4) fed straight from the registers, with each sub-block's own cumsum, so that no
//     factor exceeds e^80;
//   * the cross-sub-block terms use factors <= 1 only: with Kb_0 = e^{G_15 - G} K of sub-block 0,
//     C = Kt_1 Kb_0^T gives A_10 = Diag(beta_1) C and P_10 = Qt_1 Kb_0^T, on fp16 16x16x32
//     MFMAs (fp16 operands, as the state pass uses them);
//   * T' of the record is block lower-triangular: T'_00 and T'_11 by forward substitution; its
//     lower-left block T'_10 = -T'_11 C T'_00 is never formed -- the record keeps -C and the state
//     pass applies it as W_1 = T'_11 (X_1 - C W_0);
//   * the record's Kt_1 and Qt_1 are scaled by sub-block 0's e^{G_15} (from the record's first
//     token) and its Kb_0 by sub-block 1's (to the record's last token).
// Kt and Qt leave as whole 1 KB wave stores from registers; Kb^T (channel-major) goes through LDS.
// Occupancy hint: three waves per SIMD fit the register budget with a 16-bit g or z; an fp32 g
// or z tile holds twice the registers and two fit.  NT: the record stores carry the non-temporal
// hint (set when the records outgrow the last-level cache, so that no later pass finds them there).
template <bool NT>
__device__ __forceinline__ void rec_store16(uint8_t* dst, uint4 v) {
    if constexpr (NT) __builtin_nontemporal_store(__builtin_bit_cast(u32x4nt, v), reinterpret_cast<u32x4nt*>(dst));
    else *reinterpret_cast<uint4*>(dst) = v;
}

template <int DK, int GDT, bool GATE, bool NT>
__global__ void __launch_bounds__(64, GDT == KDA_BF16 ? 3 : 2)
chunk_intra_tok_kernel(ChunkArgs p, int64_t nslots, uint8_t* ws) {
    using R = Rec<DK, false>;
    constexpr int TOKR = R::TOK;          // tokens per record: two sub-blocks
    constexpr int KS = DK / 32;           // 32-channel groups
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int TAIL = 2 * R::TB;       // T' and P tiles, staged together

    constexpr int PH = DK / 64;           // 64-channel phases: one 128-byte line of a bf16 row
    constexpr int GSZ = (GDT == KDA_F32) ? 4 : 2;
    constexpr int CPR = 64 * 2 / 16;      // 16-byte chunks per row of a bf16 phase tile
    constexpr int CPRG = 64 * GSZ / 16;   // ... of the g / z phase tile
    constexpr int TB = TOKR * 64 * 2;     // bytes of a bf16 phase tile
    constexpr int TBG = TOKR * 64 * GSZ;  // bytes of the g / z phase tile
    constexpr int PB = 2 * TB + TBG;      // bytes of one phase's inputs: k, q, g / z
    // Inputs arrive by direct-to-LDS loads, whole lines per instruction, into [32][64]-channel
    // phase tiles whose 16-byte chunks are XOR-swizzled by row: slot(r, c) = r * CPR + (c ^ r').
    // Each lane then reads its own channels without bank conflicts.
    __shared__ __attribute__((aligned(16))) uint8_t sIn[PB];          // one phase's tiles
    __shared__ __attribute__((aligned(16))) uint16_t sKb[2 * BLK * 32];  // Kb^T of one group, fragKb
    __shared__ __attribute__((aligned(16))) float sRate[2][GATE ? DK : 4];   // gate rates: hi, lo
    __shared__ float sBeta[TOKR];
    // After the last group the input tiles are dead and hold A_00, A_11 in fp32 (for the
    // substitutions), then the staged T' / -C and P tiles (fp16).
    constexpr int O_TAIL = 2048;
    static_assert(O_TAIL + TAIL <= PB, "staging fits the input tiles");
    float (*const sA)[16][16] = reinterpret_cast<float (*)[16][16]>(sIn);
    uint8_t* const sTail = sIn + O_TAIL;

    const int lane = threadIdx.x;
    const int m = lane & 15, q = lane >> 4;

    const int64_t H = p.H;
    const int64_t gu = global_unit(p, blockIdx.x);
    const int64_t slot = gu / H;
    const int h = static_cast<int>(gu % H);
    int n;
    int64_t j0, bos, len;
    if (!locate_slot<TOKR>(p, slot, n, j0, bos, len)) return;
    const int64_t t0 = TOKR * j0;
    const int nt = static_cast<int>((len - t0) < TOKR ? (len - t0) : TOKR);
    uint8_t* rec = ws + (static_cast<int64_t>(h) * nslots + slot) * R::BYTES;
    const float keep[2] = {m < nt ? 1.f : 0.f, 16 + m < nt ? 1.f : 0.f};   // the lane's tokens exist

    // ---- beta and A into registers, then every phase's tiles; beta and the gate rates go to LDS
    // afterwards (the compiler counts its own waits for them, and the per-phase waits below only
    // need the older tile transfers done).  Rows past the record's last token read zeros: the
    // buffer ranges end there.
    const int64_t row0 = (bos + t0) * H + h;
    float av[GATE ? DK / 64 : 1];
    // beta of token `lane`: lanes 32 .. 63 and tokens past the record fall outside the range
    const float bval = bf16_val(__builtin_amdgcn_raw_buffer_load_b16(
        make_rsrc(static_cast<const uint16_t*>(p.beta) + row0, nt * static_cast<uint32_t>(H) * 2),
        lane * static_cast<uint32_t>(H) * 2, 0, 0));
    if constexpr (GATE) {
#pragma unroll
        for (int i = 0; i < DK / 64; ++i) av[i] = p.gate_A[static_cast<int64_t>(h) * DK + 64 * i + lane];
    }
    __builtin_amdgcn_sched_barrier(0);   // these loads stay older than the tile transfers
    const uint32_t rowb = static_cast<uint32_t>(H * DK * 2);                     // bytes per token
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(static_cast<const uint16_t*>(p.k) + row0 * DK, nt * rowb);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(static_cast<const uint16_t*>(p.q) + row0 * DK, nt * rowb);
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(static_cast<const uint8_t*>(p.g) + row0 * DK * GSZ,
                                                nt * rowb / 2 * GSZ);
    // phase ph's k, q and g / z tiles into sIn: 1 KB per wave instruction, eight or sixteen rows
    // of whole lines, non-temporal (each input is read once)
    auto load_phase = [&](int ph) {
#pragma unroll
        for (int u = 0; u < TB / 1024; ++u) {
            const int S = 64 * u + lane, rr = S / CPR, c = (S % CPR) ^ (rr & (CPR - 1));
            const uint32_t off = rr * rowb + ph * 128 + 16 * c;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(sIn + 1024 * u),
                                                     16, off, 0, 0, CP_NT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (__attribute__((address_space(3))) void*)(sIn + TB + 1024 * u),
                                                     16, off, 0, 0, CP_NT);
        }
#pragma unroll
        for (int u = 0; u < TBG / 1024; ++u) {
            const int S = 64 * u + lane, rr = S / CPRG, c = (S % CPRG) ^ (rr & (CPRG - 1));
            const uint32_t off = rr * (rowb / 2 * GSZ) + ph * 64 * GSZ + 16 * c;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (__attribute__((address_space(3))) void*)(sIn + 2 * TB + 1024 * u),
                                                     16, off, 0, 0, CP_NT);
        }
    };
    load_phase(0);
    if (lane < TOKR) sBeta[lane] = bval;
    if constexpr (GATE) {   // one rate per (head, channel), shared through LDS
#pragma unroll
        for (int i = 0; i < DK / 64; ++i) {
            const GateRate gr = gate_rate(av[i]);
            sRate[0][64 * i + lane] = gr.hi;
            sRate[1][64 * i + lane] = gr.lo;
        }
    }
    // token m of sub-block s: its four channels 32 lk + 16 hf + 4 q .. + 3 of phase tile `tile`
    // (bf16: 8 bytes)
    auto tile_bf16 = [&](const uint8_t* tile, int s, int lk, int hf) -> uint2 {
        const int r = 16 * s + m, byte = (32 * lk + 16 * hf + 4 * q) * 2, c = byte >> 4;
        return *reinterpret_cast<const uint2*>(tile + (r * CPR + (c ^ (r & (CPR - 1)))) * 16 + (byte & 15));
    };
    auto tile_f32 = [&](const uint8_t* tile, int s, int lk, int hf) -> uint4 {
        const int r = 16 * s + m, c = 8 * lk + 4 * hf + q;
        return *reinterpret_cast<const uint4*>(tile + (r * CPRG + (c ^ (r & (CPRG - 1)))) * 16);
    };
    auto raw16 = [](const uint32_t* w, int j) -> float {      // element j of packed bf16 words
        return (j & 1) ? __uint_as_float(w[j >> 1] & 0xffff0000u) : __uint_as_float(w[j >> 1] << 16);
    };
    wave_fence();   // beta and the gate rates are read across lanes

    // Per 32-channel group, both sub-blocks side by side: the gate and the scans, the factors,
    // the G_15 broadcasts (LDS swizzles) issued together, the MFMAs, then Kb.
    f32x4 accA[2] = {zero4(), zero4()}, accP[2] = {zero4(), zero4()}, accC = zero4(), accQ = zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int ph = kk >> 1, lk = kk & 1;
        if (lk == 0) {   // this phase's tiles have landed
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            wave_fence();
        }
        const uint8_t* tk = sIn;
        uint32_t rk[2][4], rq[2][4], rg[2][2 * (GSZ / 2) * 2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const uint2 a = tile_bf16(tk, s, lk, hf), b = tile_bf16(tk + TB, s, lk, hf);
                rk[s][2 * hf] = a.x; rk[s][2 * hf + 1] = a.y;
                rq[s][2 * hf] = b.x; rq[s][2 * hf + 1] = b.y;
                if constexpr (GSZ == 4) {
                    const uint4 g4 = tile_f32(tk + 2 * TB, s, lk, hf);
                    rg[s][4 * hf] = g4.x; rg[s][4 * hf + 1] = g4.y; rg[s][4 * hf + 2] = g4.z; rg[s][4 * hf + 3] = g4.w;
                } else {
                    const uint2 g2 = tile_bf16(tk + 2 * TB, s, lk, hf);
                    rg[s][2 * hf] = g2.x; rg[s][2 * hf + 1] = g2.y;
                }
            }
        if (lk == 1 && ph + 1 < PH) {
            // the phase's tiles are read: the next phase's transfers overwrite them while this
            // group computes
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the tile reads above are done
            wave_fence();
            load_phase(ph + 1);
        }
        float x[2][8], e1[2][8], gm[2][8];
        float4 rate[2][2];   // [hi, lo][channel half]
        if constexpr (GATE) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                rate[w][0] = *reinterpret_cast<const float4_ma*>(&sRate[w][32 * kk + 4 * q]);
                rate[w][1] = *reinterpret_cast<const float4_ma*>(&sRate[w][32 * kk + 16 + 4 * q]);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // g of token m (0 past the record's tokens, as in the unfused path's zero fill)
                float gv;
                if constexpr (GATE) {
                    const float z = (GDT == KDA_F32) ? __uint_as_float(rg[s][j]) : raw16(rg[s], j);
                    auto pick = [&](const float4& r4) {
                        return (j & 3) == 0 ? r4.x : (j & 3) == 1 ? r4.y : (j & 3) == 2 ? r4.z : r4.w;
                    };
                    gv = gate_log_decay(pick(rate[0][j >> 2]), pick(rate[1][j >> 2]), z, p.g_min) * keep[s];
                } else if constexpr (GDT == KDA_F32) {
                    gv = __uint_as_float(rg[s][j]);
                } else {
                    gv = raw16(rg[s], j);
                }
                x[s][j] = gv * LOG2E;
            }
        // inclusive cumsum over the 16 tokens of each row and sub-block (log2 units): a
        // Hillis-Steele scan
#define KDA_SCAN_STEP(CTRL)                                                                          \
        _Pragma("unroll") for (int s = 0; s < 2; ++s)                                              \
        _Pragma("unroll") for (int j = 0; j < 8; ++j)                                              \
            x[s][j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[s][j]), CTRL, 0xf, 0xf, true));
        KDA_SCAN_STEP(0x111)
        KDA_SCAN_STEP(0x112)
        KDA_SCAN_STEP(0x114)
        KDA_SCAN_STEP(0x118)
#undef KDA_SCAN_STEP
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) e1[s][j] = fexp2(x[s][j]);         // e^{G} <= 1
        // e^{G_15}: lane 15 of the row (bitmask swizzle: lane -> (lane & 16) | 15)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                gm[s][j] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(e1[s][j]), 0x1F0));
        // sub-block 0: Kt, Qt, Kd with its own cumsum; Kb_0 = Kd e^{G_15} <= 1 is kept for the
        // cross products
        float kb0[8];
        {
            float kt[8], qt[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float kv = raw16(rk[0], j), qv = raw16(rq[0], j);
                kt[j] = kv * e1[0][j];
                qt[j] = qv * (e1[0][j] * p.scale);                       // the output scale rides on Qt and P
                const float kd = kv * fexp2(-x[0][j]);                   // e^{-G} <= e^80
                accA[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[j], kd, accA[0], 0, 0, 0);
                accP[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt[j], kd, accP[0], 0, 0, 0);
                kb0[j] = kd * gm[0][j];
            }
            // Kt is stored negated: the state passes form V - Kt S as one product onto V
            rec_store16<NT>(rec + (64 * kk + lane) * 16,
                            make_uint4(f16_pair(-kt[0], -kt[1]), f16_pair(-kt[2], -kt[3]),
                                       f16_pair(-kt[4], -kt[5]), f16_pair(-kt[6], -kt[7])));
            rec_store16<NT>(rec + R::OFF_QT0 + (64 * kk + lane) * 16,
                            make_uint4(f16_pair(qt[0], qt[1]), f16_pair(qt[2], qt[3]),
                                       f16_pair(qt[4], qt[5]), f16_pair(qt[6], qt[7])));
        }
        // sub-block 1: the same with its own cumsum, plus C = Kt_1 Kb_0^T and Qt_1 Kb_0^T; the
        // record holds Kt_1, Qt_1 scaled from the record's first token
        {
            float kt[8], qt[8], kb1[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float kv = raw16(rk[1], j), qv = raw16(rq[1], j);
                kt[j] = kv * e1[1][j];
                qt[j] = qv * (e1[1][j] * p.scale);
                const float kd = kv * fexp2(-x[1][j]);
                accA[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[j], kd, accA[1], 0, 0, 0);
                accP[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt[j], kd, accP[1], 0, 0, 0);
                kb1[j] = kd * gm[1][j];
            }
            // the cross products on one fp16 MFMA each: slot j of a lane is the same channel in
            // both operands, and the record keeps these factors in fp16 anyway
            f16x8 k1h, q1h, b0h;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                k1h[j] = static_cast<_Float16>(kt[j]);
                q1h[j] = static_cast<_Float16>(qt[j]);
                b0h[j] = static_cast<_Float16>(kb0[j]);
            }
            accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1h, b0h, accC, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(q1h, b0h, accQ, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                kt[j] *= gm[0][j];
                qt[j] *= gm[0][j];
            }
            rec_store16<NT>(rec + R::OFF_KT1 + (64 * kk + lane) * 16,
                            make_uint4(f16_pair(-kt[0], -kt[1]), f16_pair(-kt[2], -kt[3]),
                                       f16_pair(-kt[4], -kt[5]), f16_pair(-kt[6], -kt[7])));
            rec_store16<NT>(rec + R::OFF_QT1 + (64 * kk + lane) * 16,
                            make_uint4(f16_pair(qt[0], qt[1]), f16_pair(qt[2], qt[3]),
                                       f16_pair(qt[4], qt[5]), f16_pair(qt[6], qt[7])));
            // Kb^T of both sub-blocks, staged in fragKb order (Kb_0 scaled to the record's last
            // token).  The group's two tiles hold 64 16-byte slots each; slot L sits at
            // L ^ ((L >> 3) & 7), which spreads each write instruction over twice the banks.
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * kk + 16 * (j >> 2) + 4 * q + (j & 3);
                const int L = (c & 15) + 16 * (m >> 2);
                const int at = 512 * (j >> 2) + 8 * (L ^ ((L >> 3) & 7)) + (m & 3);
                sKb[at] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(kb0[j] * gm[1][j]));
                sKb[at + 4] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(kb1[j]));
            }
        }
        wave_fence();   // the group's Kb^T is read across lanes, then leaves as two 1 KB stores
        {
            const int src = 16 * (lane ^ ((lane >> 3) & 7));
            uint8_t* const dst = rec + R::kb_off(2 * kk) + 16 * lane;
            const uint8_t* const kb = reinterpret_cast<const uint8_t*>(sKb);
            rec_store16<NT>(dst, *reinterpret_cast<const uint4_ma*>(kb + src));
            rec_store16<NT>(dst + 1024, *reinterpret_cast<const uint4_ma*>(kb + 1024 + src));
        }
        if (m == 15) {   // e^{G_31} - 1 per channel: the product of the sub-blocks' e^{G_15}
            float* gp = reinterpret_cast<float*>(rec + R::OFF_G) + 32 * kk + 4 * q;
            float d[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) d[j] = fmaf(gm[0][j], gm[1][j], -1.f);
            *reinterpret_cast<float4*>(gp) = make_float4(d[0], d[1], d[2], d[3]);
            *reinterpret_cast<float4*>(gp + 16) = make_float4(d[4], d[5], d[6], d[7]);
        }
    }

    // ---- A_00, A_11 to LDS (for the substitutions); -C and P staged in fp16.  Lane (m, q) holds
    // rows 4q + i of column m.  Staged tiles: T'_00, -C, T'_11, then P_00, P_10, P_11.
    uint16_t* const tT = reinterpret_cast<uint16_t*>(sTail);
    uint16_t* const tP = reinterpret_cast<uint16_t*>(sTail + R::TB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * q + i, sc = m;
        sA[0][r][sc] = (sc < r) ? accA[0][i] * sBeta[r] : 0.f;
        sA[1][r][sc] = (sc < r) ? accA[1][i] * sBeta[16 + r] : 0.f;
        tT[256 + fragT(r, sc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-accC[i]));
        tP[fragT(r, sc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>((sc <= r) ? accP[0][i] : 0.f));
        tP[256 + fragT(r, sc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(accQ[i]));
        tP[512 + fragT(r, sc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>((sc <= r) ? accP[1][i] : 0.f));
    }
    wave_fence();   // sA and sBeta are read across lanes below

    // ---- T'_ss = (I + A_ss)^{-1} Diag(beta_s): forward substitution, lane 16 s + j = column j of
    // sub-block s
    if (lane < 32) {
        const int sb = lane >> 4, jc = lane & 15;
        float (*const A)[16] = sA[sb];
        float t[16];
        float4 nxt[4], cur[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) nxt[u] = *reinterpret_cast<const float4_ma*>(&A[1][4 * u]);
        t[0] = (jc == 0) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
#pragma unroll
            for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
            if (r + 1 < 16) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (4 * u < r + 1) nxt[u] = *reinterpret_cast<const float4_ma*>(&A[r + 1][4 * u]);
            }
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < r; ++sp) {
                const float4& c4 = cur[sp >> 2];
                const float a = (sp & 3) == 0 ? c4.x : (sp & 3) == 1 ? c4.y : (sp & 3) == 2 ? c4.z : c4.w;
                part[sp & 3] += a * t[sp];
            }
            t[r] = ((r == jc) ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
        }
        const float bj = sBeta[16 * sb + jc];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            tT[512 * sb + fragT(r, jc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(t[r] * bj));
    }
    wave_fence();   // T', -C and P staged
    for (int u = lane; u < TAIL / 16; u += 64)
        rec_store16<NT>(rec + (16 * u < R::TB ? R::OFF_T : R::OFF_P - R::TB) + 16 * u,
                        *reinterpret_cast<const uint4_ma*>(sTail + 16 * u));
}

// ============================================================================================
// 2. state-passing kernel: one workgroup of NW computing waves per (sequence, head, 16 NW state
//    columns), plus NW waves that only issue its transfers when NW <= 2
// ============================================================================================

// Long sequences in the two-kernel path: segments of 2^SEG_SHIFT tokens (kda_chunk_util.hpp).
constexpr int SEG_SHIFT = 13;
constexpr int64_t SEG_TOK = int64_t(1) << SEG_SHIFT;
constexpr int SEG_MAX_SEQS = 128;   // segmented launches have at most 128 sequences (use_segments)

// MODE 0: whole sequences.  MODE 1: segment pass 1.  MODE 2: segment pass 2.
template <int DK, int IDT, int ODT, bool PRECISE, int NW, bool CKPT, int MODE>
__global__ void __launch_bounds__(64 * (NW + state_helpers(NW)), 1) chunk_state_kernel(ChunkArgs p, int32_t n_vblk,
                                                                 int64_t nslots, const uint8_t* ws,
                                                                 SegArgs sg) {
    using R = Rec<DK, PRECISE>;
    constexpr int KS = DK / 32;
    constexpr int CT = DK / 16;
    constexpr int NB = 2;                              // records per streamed chunk
    constexpr int CHT = NB * R::TOK;                   // tokens per chunk: 64 fast, 32 precise
    constexpr int OST = R::TOK / 4;                    // o stores per lane and record
    constexpr int ESZ = (IDT == KDA_F32) ? 4 : 2;
    constexpr int OSZ = (ODT == KDA_F32) ? 4 : 2;
    constexpr int WKB = 64 * 16;                       // bytes one wave moves per DMA load
    constexpr int ROUNDS = (NB * R::BYTES + NW * WKB - 1) / (NW * WKB);
    constexpr int RBYTES = ROUNDS * NW * WKB;          // a chunk's records, padded to whole rounds
    constexpr int BVW = 16 * NW;                       // state columns per workgroup
    constexpr int VROW = BVW * ESZ;                    // bytes of one token's V slice
    constexpr int VROUNDS = (CHT * VROW + NW * WKB - 1) / (NW * WKB);
    constexpr int LBYTES = RBYTES + VROUNDS * NW * WKB;   // records, then V [CHT][BVW]
    constexpr int E2 = 2 * R::E;                       // bytes of one 16-bit operand array
    static_assert(WKB % VROW == 0, "a DMA round covers whole V rows");

    // Two chunk buffers.  The loop below is unrolled by two so that every access names its
    // buffer statically: the compiler then knows the records streaming into one buffer do not
    // alias the reads of the other and inserts no waits for them.
    __shared__ __attribute__((aligned(16))) uint8_t bufA[LBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t bufB[LBYTES];
    // waves 0 .. NW - 1 compute; waves NW .. NW + NH - 1 (NH = NW or 0) issue the transfers and,
    // from a two-chunk LDS stage the computing waves write o into, the o stores
    constexpr int NH = state_helpers(NW);
    constexpr int OROW = BVW * OSZ;                    // bytes of one token's o slice
    constexpr int OSTAGE = CHT * OROW;                 // one chunk's o slice
    __shared__ __attribute__((aligned(16))) uint8_t ostage[NH > 0 ? 2 * OSTAGE : 16];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ln = lane & 15, lq = lane >> 4;
    const bool helper = NH > 0 && wave >= NW;
    const int dwave = NH > 0 ? wave - NW : wave;       // the transfer share of an issuing wave

    // Workgroup -> (unit, column block).  The column blocks of one unit sit 8 workgroup ids
    // apart so they land on the same XCD and share its L2 for the unit's records.  A unit is a
    // (sequence, head), or a (segment slot, head) in the segment passes; pass 1 puts the M column
    // blocks first.
    const int64_t H = p.H;
    const int64_t units = (MODE == 0 ? static_cast<int64_t>(p.n_seqs) : sg.slots) * p.heads;
    const int nvx = MODE == 1 ? sg.n_vblk_m + n_vblk : n_vblk;
    const int64_t bid = blockIdx.x;
    const int64_t grp = bid / (8 * nvx), remv = bid % (8 * nvx);
    int vb = static_cast<int>(remv / 8);
    const int64_t lu = grp * 8 + remv % 8;
    if (lu >= units) return;
    const int64_t unit = global_unit(p, lu);
    const int h = static_cast<int>(unit % H);
    int n = static_cast<int>(unit / H);
    int64_t seg = 0, seg_slot = 0;
    if constexpr (MODE == 1) {
        if (!locate_seg(p, sg, unit / H, n, seg)) return;
        seg_slot = unit / H;
    } else if constexpr (MODE == 2) {
        // every segment of the batch runs here, longest first: the full segments, then the
        // sequences' last segments by decreasing length (ranked only by the workgroups that run
        // one of those)
        __shared__ int last_order[SEG_MAX_SEQS];
        const int* order = nullptr;
        if (p.cu && p.n_seqs <= SEG_MAX_SEQS && p.n_seqs <= static_cast<int>(blockDim.x) &&
            unit / H >= full_seg_count(p, sg)) {
            rank_last_segments(p, sg, last_order);
            order = last_order;
        }
        if (!locate_seg_lpt(p, sg, unit / H, n, seg, seg_slot, order)) return;
    }
    const int DV = p.dv;
    const int32_t vstride = static_cast<int32_t>(H) * DV;

    int64_t bos, len, base;
    if (p.cu) {
        int64_t end;
        seq_bounds(p, n, bos, end);
        len = end - bos;
        base = bos / R::TOK + n;
    } else {
        bos = static_cast<int64_t>(n) * p.T;
        len = p.T;
        base = static_cast<int64_t>(n) * ((p.T + R::TOK - 1) / R::TOK);
    }
    const uint8_t* recs = ws + (static_cast<int64_t>(h) * nslots + base) * R::BYTES;

    // What this workgroup does: the chunks it runs, where its state starts and ends, and whether
    // it reads V and writes o.  A pair column block (role M) starts from the identity with V = 0.
    const int64_t nchunks_all = (len + CHT - 1) / CHT;
    int64_t c_begin = 0, c_end = nchunks_all;
    const int64_t useq = static_cast<int64_t>(n) * H + h;           // (sequence, head)
    const float* init = p.h0 ? p.h0 + useq * DK * DV : nullptr;       // nullptr: zeros
    float* fin = p.hT ? p.hT + useq * DK * DV : nullptr;              // nullptr: not stored
    int ldst = DV;                                                     // row stride of init / fin
    bool ident = false, use_v = true, emit_o = true;
    if constexpr (MODE != 0) {
        const int64_t SEGC = (int64_t(1) << sg.seg_shift) / CHT;
        const int64_t nseg = seg_count(len, sg.seg_shift);
        const int64_t us = seg_slot * H + h;                            // (segment slot, head)
        c_begin = seg * SEGC;
        c_end = c_begin + SEGC < nchunks_all ? c_begin + SEGC : nchunks_all;
        if (MODE == 1) {
            if (seg == 0) {
                if (vb >= n_vblk) return;
                if (nseg > 1) fin = sg.S + (us + H) * DK * DV;         // start of segment 1
            } else if (seg + 1 < nseg) {
                init = nullptr;
                emit_o = false;
                if (vb < sg.n_vblk_m) {
                    ident = true;
                    use_v = false;
                    fin = sg.M + us * DK * DK;
                    ldst = DK;
                } else {
                    vb -= sg.n_vblk_m;
                    fin = sg.B + us * DK * DV;
                }
            } else {
                return;                                                // the last segment: pass 2
            }
        } else {
            if (seg == 0 && !sg.from0) return;                         // ran in pass 1
            if (seg > 0) init = sg.S + us * DK * DV;                   // else the initial state
            if (seg + 1 < nseg) fin = nullptr;                         // its end state is known
        }
    }
    const int n0 = vb * BVW + wave * 16;               // this wave's first state column

    // state tiles: lane (ln, lq) of tile i holds S[16i + 4lq + r][n0 + ln]
    f32x4 S[CT];

    // Checkpoints (CKPT): the state after every ckpt_every tokens of the sequence goes to slot
    // ck_base + j - 1 (j = 1, 2, ...): ck_base = n * floor(T / every) for fixed-length batches,
    // floor(cu[n] / every) + n for packed ones (disjoint for the same reason as the block slots).
    const int64_t ck_every = CKPT ? p.ckpt_every : 1;
    const int64_t ck_base = !CKPT ? 0
                            : p.cu ? bos / ck_every + n
                                   : static_cast<int64_t>(n) * (p.T / ck_every);
    auto checkpoint = [&](int64_t done) {          // `done` tokens of the sequence processed
        if constexpr (!CKPT) return;
        if (helper || !emit_o || done > len || done % ck_every != 0) return;
        const int64_t slot = ck_base + done / ck_every - 1;
        if (slot >= p.ckpt_slots) return;
        float* dst = p.ckpt + (slot * H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < CT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[static_cast<int64_t>(16 * i + 4 * lq + r) * DV + n0 + ln] = S[i][r];
    };
    if (!helper) {
        // an absent initial state is an empty range: every load reads 0
        const __amdgpu_buffer_rsrc_t h0r =
            make_rsrc(init, init ? static_cast<uint32_t>(DK * ldst * 4) : 0u);
#pragma unroll
        for (int i = 0; i < CT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                S[i][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    h0r, ((16 * i + 4 * lq + r) * ldst + n0 + ln) * 4, 0, 0));
                if (ident) S[i][r] = (16 * i + 4 * lq + r == n0 + ln) ? 1.f : 0.f;
            }
    }

    auto tokens_in = [&](int64_t c) -> int {            // tokens of chunk c (0 past the end)
        const int64_t rem = len - c * CHT;
        return static_cast<int>(rem < 0 ? 0 : rem < CHT ? rem : CHT);
    };
    // o stores: a computing wave's store covers 32 (bf16) or 64 bytes of a row, a helper's 16 of
    // the workgroup's row slice.  When the workgroup holds every column of the state (8 waves at
    // d_v = 128) its waves' partial lines merge in L2 under the default cache policy
    // (non-temporal stores wrote 26% more bytes there and made segment pass 2 10% slower);
    // narrower workgroups, whose lines are completed by other CUs, measured 5% faster with
    // non-temporal stores.
    constexpr int O_AUX = (16 * NW >= 128) ? 0 : CP_NT;
    // helpers: chunk cp's o slice from the stage, 16 bytes a lane (OROW / 16 lanes a row); rows
    // past the chunk's tokens fall outside the range
    constexpr int OPIECE = CHT * OROW / 16;
    constexpr int OSTORES = NH > 0 ? OPIECE / (64 * NH) : 0;   // store instructions per helper
    static_assert(NH == 0 || OPIECE % (64 * NH) == 0, "whole store rounds");
    auto store_stage = [&](int64_t cp) {
        const int ntp = tokens_in(cp);
        const __amdgpu_buffer_rsrc_t orr =
            make_rsrc(static_cast<char*>(p.o) + ((bos + cp * CHT) * H + h) * DV * OSZ,
                      emit_o ? static_cast<uint32_t>(ntp * vstride * OSZ) : 0u);
        const uint8_t* const st = ostage + (cp & 1) * OSTAGE;
#pragma unroll
        for (int k = 0; k < OSTORES; ++k) {
            const int q = (k * NH + dwave) * 64 + lane;
            const int row = q / (OROW / 16), piece = q % (OROW / 16);
            typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v val = *reinterpret_cast<const u32x4v*>(st + row * OROW + 16 * piece);
            __builtin_amdgcn_raw_buffer_store_b128(val, orr, (row * vstride + vb * BVW) * OSZ + 16 * piece, 0, O_AUX);
        }
    };
    // Chunk c's records and its V slice go straight from memory into an LDS buffer (records past
    // the sequence's last block, V rows past its last token, and the padding read as zeros:
    // identity steps).  The transfers are issued in NSLICE slices at the chunk's issue points:
    // point 2b is the start of block b, point 2b + 1 its end before its o stores.  A wave issues
    // one slice at a point, since a long run of transfers stalls it until the memory pipeline
    // takes them (at two waves per workgroup, 30 transfers held each wave for a quarter of the
    // chunk).
    constexpr int NITEM = ROUNDS + VROUNDS;
    constexpr int NSLICE = NH > 0 ? 1 : STATE_SLICES;
    static_assert(NSLICE <= 2 * NB, "issue points of a chunk");
    auto prefetch_slice = [&](uint8_t* buf, int64_t c, int slice) {
        const int nt = tokens_in(c);
        const int nbk = (nt + R::TOK - 1) / R::TOK;
        const __amdgpu_buffer_rsrc_t rr =
            make_rsrc(nt > 0 ? recs + c * NB * R::BYTES : ws, static_cast<uint32_t>(nbk * R::BYTES));
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(
            nt > 0 ? static_cast<const uint8_t*>(p.v) + ((bos + c * CHT) * H + h) * DV * ESZ : p.v,
            use_v ? static_cast<uint32_t>(nt * vstride * ESZ) : 0u);
        const int i0 = slice * NITEM / NSLICE, i1 = (slice + 1) * NITEM / NSLICE;
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            if (it < i0 || it >= i1) continue;
            if (it < ROUNDS) {
                const int u = it * NW + dwave;          // this wave's 1 KB unit of the records
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rr, (__attribute__((address_space(3))) void*)(buf + u * WKB), 16,
                    u * WKB + 16 * lane, 0, 0, 0);
            } else {
                const int u = (it - ROUNDS) * NW + dwave;  // this wave's 1 KB unit of V
                const int byte = u * WKB + 16 * lane;     // within the [CHT][BVW] slice
                const int row = byte / VROW, col = byte % VROW;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    vr, (__attribute__((address_space(3))) void*)(buf + RBYTES + u * WKB), 16,
                    row * vstride * ESZ + vb * VROW + col, 0, 0, CP_NT);
            }
        }
    };

    // One chunk: NB state steps from the records in `buf` (32 tokens each fast, 16 precise).
    auto run = [&](const uint8_t* buf, int64_t c, uint8_t* nbuf) {
        const int nt = tokens_in(c);
        // memory instructions keep their order across an issue point (the end-of-chunk wait
        // counts the o stores issued after the last slice)
        auto issue_at = [&](int k) {
            if constexpr (NH == 0) {
                __builtin_amdgcn_sched_barrier(0x78F);
                if (k < NSLICE) prefetch_slice(nbuf, c + 1, k);
                __builtin_amdgcn_sched_barrier(0x78F);
            }
        };
        // per-lane bases: fragment rows, 8-byte fragments, the decay vector, this lane's V column
        const uint8_t* const l16 = lds_at(buf, 16 * lane);
        const uint8_t* const l8 = lds_at(buf, 8 * lane);
        const float* const lg = reinterpret_cast<const float*>(lds_at(buf, R::OFF_G + 16 * lq));
        const uint8_t* const lv = lds_at(buf, RBYTES + ESZ * (4 * lq * BVW + 16 * wave + ln));
        // o rows of this chunk and head; rows past the chunk's tokens fall outside the range
        const __amdgpu_buffer_rsrc_t orr =
            make_rsrc(static_cast<char*>(p.o) + ((bos + c * CHT) * H + h) * DV * OSZ,
                      emit_o ? static_cast<uint32_t>(nt * vstride * OSZ) : 0u);
        auto store_o = [&](const f32x4& O, int row0) {   // rows row0 + 4 lq + i of the chunk
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (NH > 0) {                  // into the stage (the helpers store it)
                    const int e = (row0 + 4 * lq + i) * BVW + 16 * wave + ln;
                    uint8_t* const st = ostage + (c & 1) * OSTAGE;
                    if constexpr (ODT == KDA_F32) reinterpret_cast<float*>(st)[e] = O[i];
                    else reinterpret_cast<uint16_t*>(st)[e] = bf16_bits(O[i]);
                } else {
                    const int off = ((row0 + 4 * lq + i) * vstride + n0 + ln) * OSZ;
                    if constexpr (ODT == KDA_F32)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[i]), orr, off, 0, O_AUX);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(O[i]), orr, off, 0, O_AUX);
                }
            }
        };
        auto v_rows = [&](int row0) -> f32x4 {   // V, rows as store_o
            f32x4 X;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ve = (row0 + i) * BVW;            // V[row0 + 4 lq + i][16 wave + ln]
                X[i] = (ESZ == 4) ? reinterpret_cast<const float*>(lv)[ve]
                                  : bf16_val(reinterpret_cast<const uint16_t*>(lv)[ve]);
            }
            return X;
        };
        auto v_minus = [&](const f32x4& Y, int row0) -> f32x4 {   // V - Y
            const f32x4 V = v_rows(row0);
            f32x4 X;
#pragma unroll
            for (int i = 0; i < 4; ++i) X[i] = V[i] - Y[i];
            return X;
        };
        // The Kt / Qt fragments of record b + 1 are read from LDS while record b computes (they
        // are needed first thing in a step); the rest of a record's operands are read at its
        // start and consumed later in it.  Fast: Kt_0, Qt_0, Kt_1, Qt_1; precise: Kt hi, lo, Qt
        // hi, lo.
        using FragA = typename std::conditional<PRECISE, bf16x8, f16x8>::type;
        constexpr int NFA = 4;
        FragA fa[NFA][KS], fn[NFA][KS];
        auto load_fa = [&](int b, FragA (&f)[NFA][KS]) {     // record b of the chunk
#pragma unroll
            for (int a = 0; a < NFA; ++a)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const int off = PRECISE ? a * E2 : R::fa_off(a);
                    f[a][kk] = *reinterpret_cast<const FragA*>(l16 + b * R::BYTES + off + 1024 * kk);
                }
        };
        load_fa(0, fa);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            issue_at(2 * b);
            const int rb = b * R::BYTES;                    // the record's byte offset in the buffer
            if (b + 1 < NB) load_fa(b + 1, fn);
            const float* gam = lg + rb / 4;                 // e^{G_last} - 1, from channel 4 lq
            float4 gm[CT];
#pragma unroll
            for (int i = 0; i < CT; ++i) gm[i] = *reinterpret_cast<const float4*>(gam + 16 * i);
            if constexpr (!PRECISE) {
                // ---- one 32-token step: sub-blocks 0 and 1, S taken at the record's first token
                const uint8_t* tb = l8 + rb + R::OFF_T;   // T'_00, -C, T'_11 (fragT)
                const uint8_t* pb = l8 + rb + R::OFF_P;   // P_00, P_10, P_11
                const f16x4 t00 = *reinterpret_cast<const f16x4*>(tb);
                const f16x4 ncm = *reinterpret_cast<const f16x4*>(tb + 512);
                const f16x4 t11 = *reinterpret_cast<const f16x4*>(tb + 1024);
                const f16x4 p00 = *reinterpret_cast<const f16x4*>(pb);
                const f16x8 p1x = __builtin_shufflevector(*reinterpret_cast<const f16x4*>(pb + 512),
                                                          *reinterpret_cast<const f16x4*>(pb + 1024), 0, 1, 2, 3, 4, 5, 6, 7);
                // X_s = V_s - Kt_s S (the record holds -Kt: one product accumulated onto V; the
                // beta scaling sits in T') and O_s = Qt_s S, contracting over d_k with S packed as
                // the B operand
                f32x4 X0 = v_rows(32 * b), X1 = v_rows(32 * b + 16), O0 = zero4(), O1 = zero4();
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    f16x8 sb;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sb[i] = static_cast<_Float16>(S[2 * kk][i]);
                        sb[4 + i] = static_cast<_Float16>(S[2 * kk + 1][i]);
                    }
                    X0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[0][kk], sb, X0, 0, 0, 0);
                    X1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[2][kk], sb, X1, 0, 0, 0);
                    O0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[1][kk], sb, O0, 0, 0, 0);
                    O1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[3][kk], sb, O1, 0, 0, 0);
                }
                // W_0 = T'_00 X_0, X_1' = X_1 - C W_0, W_1 = T'_11 X_1'
                f16x4 x0, x1, w0, w1;
#pragma unroll
                for (int i = 0; i < 4; ++i) x0[i] = static_cast<_Float16>(X0[i]);
                const f32x4 W0 = __builtin_amdgcn_mfma_f32_16x16x16f16(t00, x0, zero4(), 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) w0[i] = static_cast<_Float16>(W0[i]);
                const f32x4 X1p = __builtin_amdgcn_mfma_f32_16x16x16f16(ncm, w0, X1, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) x1[i] = static_cast<_Float16>(X1p[i]);
                const f32x4 W1 = __builtin_amdgcn_mfma_f32_16x16x16f16(t11, x1, zero4(), 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) w1[i] = static_cast<_Float16>(W1[i]);
                const f16x8 wx = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
                // O += P W (P and Qt carry the output scale)
                O0 = __builtin_amdgcn_mfma_f32_16x16x16f16(p00, w0, O0, 0, 0, 0);
                O1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(p1x, wx, O1, 0, 0, 0);
                issue_at(2 * b + 1);
                store_o(O0, 32 * b);
                store_o(O1, 32 * b + 16);
                // S <- Diag(e^{G_31}) S + Kb^T W = S + Diag(e^{G_31} - 1) S + [Kb_0^T Kb_1^T] W
#pragma unroll
                for (int i = 0; i < CT; ++i) {
                    const f16x8 ka = *reinterpret_cast<const f16x8*>(l16 + rb + R::kb_off(i));
                    f32x4 acc;
                    acc[0] = fmaf(S[i][0], gm[i].x, S[i][0]); acc[1] = fmaf(S[i][1], gm[i].y, S[i][1]);
                    acc[2] = fmaf(S[i][2], gm[i].z, S[i][2]); acc[3] = fmaf(S[i][3], gm[i].w, S[i][3]);
                    S[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, wx, acc, 0, 0, 0);
                }
            } else {
                // ---- one 16-token step, split-bf16 operands
                const uint16_t* Tp = reinterpret_cast<const uint16_t*>(l8 + rb + R::OFF_T);
                const s16x4 ph = *reinterpret_cast<const s16x4*>(l8 + rb + R::OFF_P);
                const s16x4 pl = *reinterpret_cast<const s16x4*>(l8 + rb + R::OFF_P + 512);
                f32x4 Y = zero4(), O = zero4();
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    float sv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) { sv[i] = S[2 * kk][i]; sv[4 + i] = S[2 * kk + 1][i]; }
                    bf16x8 sbh, sbl;
                    split8(sv, sbh, sbl);
                    Y = mfma32_bf16_x3(fa[0][kk], fa[1][kk], sbh, sbl, Y);
                    O = mfma32_bf16_x3(fa[2][kk], fa[3][kk], sbh, sbl, O);
                }
                const f32x4 X = v_minus(Y, 16 * b);
                s16x4 xh, xl;
                split4(X, xh, xl);
                const f32x4 W = mfma16_bf16_x3(*reinterpret_cast<const s16x4*>(Tp), *reinterpret_cast<const s16x4*>(Tp + 256),
                                               xh, xl, zero4());
                s16x4 wh, wl;
                split4(W, wh, wl);
                O = mfma16_bf16_x3(ph, pl, wh, wl, O);
                issue_at(2 * b + 1);
                store_o(O, 16 * b);
                const uint8_t* kbh = l8 + rb + 4 * E2;
                const uint8_t* kbl = l8 + rb + 5 * E2;
#pragma unroll
                for (int i = 0; i < CT; ++i) {
                    const s16x4 kh = *reinterpret_cast<const s16x4*>(kbh + 512 * i);
                    const s16x4 kl = *reinterpret_cast<const s16x4*>(kbl + 512 * i);
                    f32x4 acc;
                    acc[0] = fmaf(S[i][0], gm[i].x, S[i][0]); acc[1] = fmaf(S[i][1], gm[i].y, S[i][1]);
                    acc[2] = fmaf(S[i][2], gm[i].z, S[i][2]); acc[3] = fmaf(S[i][3], gm[i].w, S[i][3]);
                    S[i] = mfma16_bf16_x3(kh, kl, wh, wl, acc);
                }
            }
            if (b + 1 < NB) {
#pragma unroll
                for (int a = 0; a < NFA; ++a)
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) fa[a][kk] = fn[a][kk];
            }
        }
    };

    // Each half-iteration runs the current chunk while the next chunk's transfers go out, then
    // waits for those transfers -- the o stores of the records from the one that issued the last
    // slice on (OST each) may stay in flight, every load is older -- and meets the other waves at
    // the barrier.
    // blocks whose o stores follow the last slice (point NSLICE - 1): b >= (NSLICE - 1) / 2
    constexpr int WAIT_LOADS = vmcnt_imm(OST * (NB - (NSLICE - 1) / 2));
    // With helpers, a helper issues all of chunk c + 1's transfers while the computing waves run
    // chunk c, then waits for them; the computing waves issue only o stores and do not wait.
    auto step = [&](const uint8_t* buf, int64_t c, uint8_t* nbuf) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NH == 0) {
            run(buf, c, nbuf);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(WAIT_LOADS);
        } else {
            if (helper) {
                // the next chunk's transfers, then the previous chunk's o; the wait leaves the
                // stores in flight (memory operations of a wave complete in issue order)
                prefetch_slice(nbuf, c + 1, 0);
                __builtin_amdgcn_sched_barrier(0x78F);
                if (c > c_begin) {
                    store_stage(c - 1);
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(OSTORES));
                } else {
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                }
            } else {
                run(buf, c, nbuf);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    if (NH == 0 || helper) {
#pragma unroll
        for (int sl = 0; sl < NSLICE; ++sl) prefetch_slice(bufA, c_begin, sl);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
    // (A checkpoint's stores go out before the next chunk's transfers, so they are older than
    // every load the waits above count on.)
    for (int64_t ci = c_begin; ci < c_end; ci += 2) {
        step(bufA, ci, bufB);
        checkpoint((ci + 1) * CHT);
        if (ci + 1 >= c_end) break;
        step(bufB, ci + 1, bufA);
        checkpoint((ci + 2) * CHT);
    }
    if (helper && c_end > c_begin) store_stage(c_end - 1);   // the last chunk's o (staged before the last barrier)

    if (fin && !helper) {
#pragma unroll
        for (int i = 0; i < CT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                fin[static_cast<int64_t>(16 * i + 4 * lq + r) * ldst + n0 + ln] = S[i][r];
    }
}

// Segment pass 1 at d_k = d_v = 128 with 16-bit inputs: one workgroup of eight waves per
// (segment, head) for every segment but a sequence's last, running the segment's pair at once --
// wave w holds state columns 16 w .. 16 w + 15 of both M (from the identity, V = 0) and B (from
// zero, with V).  The records' heads (no Qt, P: no o here) stream through LDS once, packed; the
// two tiles' dependent chains interleave in each wave.
template <int IDT>
__global__ void __launch_bounds__(512, 1) chunk_pair_kernel(ChunkArgs p, int64_t nslots, const uint8_t* ws,
                                                            SegArgs sg) {
    constexpr int DK = 128, NW = 8;
    using R = Rec<DK, false>;
    constexpr int KS = DK / 32, CT = DK / 16;
    constexpr int NB = 2, CHT = NB * R::TOK;           // two 32-token records per chunk
    constexpr int WKB = 64 * 16;
    constexpr int PREC = R::HEAD;                      // a record's head: -Kt, Kb^T, T', decay
    constexpr int RUNITS = NB * PREC / WKB;            // 1 KB units of a chunk's heads
    constexpr int ROUNDS = (RUNITS + NW - 1) / NW;
    constexpr int RBYTES = NB * PREC;                  // record b's head at b * PREC in LDS
    constexpr int BVW = 16 * NW;                       // 128 columns: all of M, all of B
    constexpr int VROW = BVW * 2;
    constexpr int VROUNDS = (CHT * VROW + NW * WKB - 1) / (NW * WKB);
    constexpr int LBYTES = RBYTES + VROUNDS * NW * WKB;
    static_assert(PREC % WKB == 0, "record heads are whole 1 KB units");
    static_assert(IDT == KDA_BF16, "16-bit inputs");
    __shared__ __attribute__((aligned(16))) uint8_t bufA[LBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t bufB[LBYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t H = p.H;
    const int64_t unit = global_unit(p, blockIdx.x);   // (segment slot, head)
    const int h = static_cast<int>(unit % H);
    int n;
    int64_t seg;
    if (!locate_seg(p, sg, unit / H, n, seg)) return;
    const int32_t vstride = static_cast<int32_t>(H) * DK;
    int64_t bos, len, base;
    if (p.cu) {
        int64_t end;
        seq_bounds(p, n, bos, end);
        len = end - bos;
        base = bos / R::TOK + n;
    } else {
        bos = static_cast<int64_t>(n) * p.T;
        len = p.T;
        base = static_cast<int64_t>(n) * ((p.T + R::TOK - 1) / R::TOK);
    }
    const int64_t nseg = seg_count(len, sg.seg_shift);
    if (seg + 1 >= nseg) return;                       // a sequence's last segment has no pair
    const uint8_t* recs = ws + (static_cast<int64_t>(h) * nslots + base) * R::BYTES;
    const int64_t SEGC = (int64_t(1) << sg.seg_shift) / CHT;
    const int64_t nchunks_all = (len + CHT - 1) / CHT;
    const int64_t c_begin = seg * SEGC;
    const int64_t c_end = c_begin + SEGC < nchunks_all ? c_begin + SEGC : nchunks_all;
    const int n0 = wave * 16;                          // this wave's first column of M and of B

    // tile 0: M (lane (ln, lq) holds M[16 i + 4 lq + r][n0 + ln]); tile 1: B, the same layout
    f32x4 S[2][CT];
#pragma unroll
    for (int i = 0; i < CT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            S[0][i][r] = (16 * i + 4 * lq + r == n0 + ln) ? 1.f : 0.f;
            S[1][i][r] = 0.f;
        }
    auto tokens_in = [&](int64_t c) -> int {
        const int64_t rem = len - c * CHT;
        return static_cast<int>(rem < 0 ? 0 : rem < CHT ? rem : CHT);
    };
    // Chunk c's record heads and its V rows into an LDS buffer: items [i0, i1) of this wave's
    // share.
    constexpr int NITEM = ROUNDS + VROUNDS;
    auto prefetch = [&](uint8_t* buf, int64_t c, int i0, int i1) {
        const int nt = tokens_in(c);
        const int nbk = (nt + R::TOK - 1) / R::TOK;
        const __amdgpu_buffer_rsrc_t rr =
            make_rsrc(nt > 0 ? recs + c * NB * R::BYTES : ws, static_cast<uint32_t>(nbk * R::BYTES));
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(
            nt > 0 ? static_cast<const uint8_t*>(p.v) + ((bos + c * CHT) * H + h) * DK * 2 : p.v,
            static_cast<uint32_t>(nt * vstride * 2));
#pragma unroll
        for (int it = 0; it < ROUNDS; ++it) {
            const int u = it * NW + wave;               // unit u % (PREC / WKB) of record u / (PREC / WKB)
            if (it < i0 || it >= i1 || u >= RUNITS) continue;
            const int src = (u / (PREC / WKB)) * R::BYTES + (u % (PREC / WKB)) * WKB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (__attribute__((address_space(3))) void*)(buf + u * WKB), 16,
                                                     src + 16 * lane, 0, 0, 0);
        }
#pragma unroll
        for (int it = 0; it < VROUNDS; ++it) {
            if (ROUNDS + it < i0 || ROUNDS + it >= i1) continue;
            const int u = it * NW + wave;
            const int byte = u * WKB + 16 * lane;
            const int row = byte / VROW, col = byte % VROW;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(buf + RBYTES + u * WKB),
                                                     16, row * vstride * 2 + col, 0, 0, CP_NT);
        }
    };
    // one chunk: two 32-token steps of both tiles
    auto run = [&](uint8_t* buf, int64_t c, uint8_t* nbuf) {
        // The next chunk's transfers: a wave issues its share at one of four points of record 0
        // (its start, after its Y products, after its W chain, after its state update), two waves
        // on different SIMDs per point.  Issued by all waves at once, the transfers fill the
        // memory pipeline and the waves stall in turn for up to a third of the chunk; staggered,
        // each wave waits only behind one other.  (Memory instructions stay at these points.)
        auto issue = [&](int k) {
            __builtin_amdgcn_sched_barrier(0x78F);
            if (k == ((wave + 2 * (wave >> 2)) & 3) && c + 1 < c_end) prefetch(nbuf, c + 1, 0, NITEM);
            __builtin_amdgcn_sched_barrier(0x78F);
        };
        // per-lane bases: fragment rows, 8-byte fragments, the decay vector, this lane's V column
        const uint8_t* const l16 = lds_at(buf, 16 * lane);
        const uint8_t* const l8 = lds_at(buf, 8 * lane);
        const float* const lg = reinterpret_cast<const float*>(lds_at(buf, R::OFF_G + 16 * lq));
        const uint16_t* const lv = lds_at(reinterpret_cast<uint16_t*>(buf + RBYTES), 2 * (4 * lq * BVW + n0 + ln));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b == 0) issue(0);
            const int rb = b * PREC;
            const float* gam = lg + rb / 4;                                   // e^{G_last} - 1
            const f16x4 t00 = *reinterpret_cast<const f16x4*>(l8 + rb + R::OFF_T);   // T'_00, -C, T'_11
            const f16x4 ncm = *reinterpret_cast<const f16x4*>(l8 + rb + R::OFF_T + 512);
            const f16x4 t11 = *reinterpret_cast<const f16x4*>(l8 + rb + R::OFF_T + 1024);
            // X_s = V_s - Kt_s S for both tiles (V = 0 for M): the record holds -Kt, so one
            // product accumulates onto V (S packed as the B operand, contraction over d_k)
            f32x4 X[2][2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                X[0][0][i] = 0.f;
                X[0][1][i] = 0.f;
                X[1][0][i] = bf16_val(lv[(32 * b + i) * BVW]);
                X[1][1][i] = bf16_val(lv[(32 * b + 16 + i) * BVW]);
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const f16x8 k0 = *reinterpret_cast<const f16x8*>(l16 + rb + 1024 * kk);
                const f16x8 k1 = *reinterpret_cast<const f16x8*>(l16 + rb + R::OFF_KT1 + 1024 * kk);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f16x8 sb;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sb[i] = static_cast<_Float16>(S[t][2 * kk][i]);
                        sb[4 + i] = static_cast<_Float16>(S[t][2 * kk + 1][i]);
                    }
                    X[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, sb, X[t][0], 0, 0, 0);
                    X[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, sb, X[t][1], 0, 0, 0);
                }
            }
            if (b == 0) issue(1);
            // W_0 = T'_00 X_0, X_1' = X_1 - C W_0, W_1 = T'_11 X_1', the two tiles' chains
            // advanced step by step so each product's latency is covered by the other tile's
            f16x4 x0[2], w0[2], x1[2], w1[2];
            f32x4 Wt[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) x0[t][i] = static_cast<_Float16>(X[t][0][i]);
#pragma unroll
            for (int t = 0; t < 2; ++t) Wt[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(t00, x0[t], zero4(), 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) w0[t][i] = static_cast<_Float16>(Wt[t][i]);
#pragma unroll
            for (int t = 0; t < 2; ++t) Wt[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(ncm, w0[t], X[t][1], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) x1[t][i] = static_cast<_Float16>(Wt[t][i]);
#pragma unroll
            for (int t = 0; t < 2; ++t) Wt[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(t11, x1[t], zero4(), 0, 0, 0);
            f16x8 wx[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) w1[t][i] = static_cast<_Float16>(Wt[t][i]);
                wx[t] = __builtin_shufflevector(w0[t], w1[t], 0, 1, 2, 3, 4, 5, 6, 7);
            }
            if (b == 0) issue(2);
            // S <- Diag(e^{G_31}) S + Kb^T W for both tiles
#pragma unroll
            for (int i = 0; i < CT; ++i) {
                const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * i);
                const f16x8 ka = *reinterpret_cast<const f16x8*>(l16 + rb + R::kb_off(i));
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x4 acc;
                    acc[0] = fmaf(S[t][i][0], gm.x, S[t][i][0]); acc[1] = fmaf(S[t][i][1], gm.y, S[t][i][1]);
                    acc[2] = fmaf(S[t][i][2], gm.z, S[t][i][2]); acc[3] = fmaf(S[t][i][3], gm.w, S[t][i][3]);
                    S[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, wx[t], acc, 0, 0, 0);
                }
            }
            if (b == 0) issue(3);
        }
    };

    prefetch(bufA, c_begin, 0, NITEM);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    for (int64_t ci = c_begin; ci < c_end; ci += 2) {
        __builtin_amdgcn_sched_barrier(0);
        run(bufA, ci, bufB);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        if (ci + 1 >= c_end) break;
        __builtin_amdgcn_sched_barrier(0);
        run(bufB, ci + 1, bufA);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
    }
    const int64_t us = unit;                           // (segment slot, head)
    float* Mo = sg.M + us * DK * DK;
    float* Bo = sg.B + us * DK * DK;
#pragma unroll
    for (int i = 0; i < CT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t e = static_cast<int64_t>(16 * i + 4 * lq + r) * DK + n0 + ln;
            Mo[e] = S[0][i][r];
            Bo[e] = S[1][i][r];
        }
}

// Segment scan: one workgroup per (sequence, head, 16 state columns) walks the sequence's
// segments, S_start(s + 1) = M_s S_start(s) + B_s for s = s0 .. nseg - 2, in fp32: s0 = 0 from
// the initial state when pass 1 made segment 0 a pair too (from0), else s0 = 1 from segment 1's
// start state, which pass 1 wrote after running segment 0 whole.  The column
// blocks are independent (M acts on the rows), so they run apart.  Each step is a d_k x d_k by
// d_k x 16 product on fp32 MFMAs (16x16x4): wave w owns output row tile w (d_k / 16 waves), B_s seeds
// the accumulators, S_start(s) is read from LDS (double-buffered, one barrier per step), and the
// M rows and B of the step after next are loaded into registers while the current step computes.
// MFMA step (m, e) of a tile contracts over the four columns 16 m + 4 c + e, c = 0..3: lane
// (i, c) supplies M[row i][16 m + 4 c + e] from its float4 of M[row i][16 m + 4 c .. + 3], and
// S_start[16 m + 4 c + e][j] for lane (j, c) comes from LDS.
constexpr int scan_waves(int dk) { return dk / 16; }   // one 16-row tile of the output per wave
template <int DK>
__global__ void __launch_bounds__(64 * scan_waves(DK)) seg_scan_kernel(ChunkArgs p, SegArgs sg) {
    constexpr int NT = DK / 16;                      // row tiles
    constexpr int NWS = scan_waves(DK);
    constexpr int TPW = NT / NWS;                    // row tiles per wave
    constexpr int NTH = 64 * NWS;
    constexpr int NM = DK / 16;                      // float4s of one M row a lane holds
    constexpr int SP = 17;                           // LDS row pitch of S_start (floats)
    __shared__ float sS[2][DK * SP];
    const int DV = p.dv, ncb = DV / 16;
    const int64_t H = p.H;
    // Workgroup -> (sequence, head) and column block: the column blocks of one (sequence, head)
    // sit 8 workgroup ids apart, so they land on one XCD and read each M_s from HBM once, the
    // others from that XCD's L2.
    const int64_t grp = blockIdx.x / (8 * ncb), rem = blockIdx.x % (8 * ncb);
    const int cb = static_cast<int>(rem / 8);
    const int64_t lu = grp * 8 + rem % 8;
    if (lu >= static_cast<int64_t>(p.n_seqs) * p.heads) return;
    const int64_t useq = global_unit(p, lu);
    const int n = static_cast<int>(useq / H), h = static_cast<int>(useq % H);
    int64_t len, slot0;
    if (p.cu) {
        int64_t bos, end;
        seq_bounds(p, n, bos, end);
        len = end - bos;
        slot0 = (bos >> sg.seg_shift) + n;
    } else {
        len = p.T;
        slot0 = static_cast<int64_t>(n) * seg_count(p.T, sg.seg_shift);
    }
    const int64_t nseg = seg_count(len, sg.seg_shift);
    const int64_t s_first = sg.from0 ? 0 : 1;         // first segment with a pair
    if (nseg < s_first + 2) return;                   // no pair before the last segment
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int li = lane & 15, lc = lane >> 4;         // row / column within a tile; K group
    auto m_of = [&](int64_t s) { return sg.M + ((slot0 + s) * H + h) * DK * DK; };
    auto b_of = [&](int64_t s) { return sg.B + ((slot0 + s) * H + h) * DK * DV + cb * 16; };

    // this lane's M values of the wave's tiles and B seeds (rows 16 r + 4 lc + v, column li), for
    // two steps: the loads run two steps ahead of the products
    float4 mrA[TPW][NM], mrB[TPW][NM];
    f32x4 brA[TPW], brB[TPW];
    auto load_step = [&](int64_t s, float4 (&mr)[TPW][NM], f32x4 (&br)[TPW]) {
        const float* M = m_of(s);
        const float* Bm = b_of(s);
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
            const int r = wave + NWS * q;
#pragma unroll
            for (int m = 0; m < NM; ++m)
                mr[q][m] = *reinterpret_cast<const float4*>(M + (16 * r + li) * DK + 16 * m + 4 * lc);
#pragma unroll
            for (int v = 0; v < 4; ++v) br[q][v] = Bm[static_cast<int64_t>(16 * r + 4 * lc + v) * DV + li];
        }
    };
    {
        // S_start(s_first): the initial state (zeros when absent) or segment 1's start from pass 1
        const float* S1 = sg.from0 ? (p.h0 ? p.h0 + useq * DK * DV + cb * 16 : nullptr)
                                   : sg.S + ((slot0 + 1) * H + h) * DK * DV + cb * 16;
        // every load first, then the LDS stores: one wait for all of them
        constexpr int PER = DK * 16 / NTH;
        float s1v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = t + NTH * i;
            s1v[i] = S1 ? S1[(e >> 4) * DV + (e & 15)] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = t + NTH * i;
            sS[0][(e >> 4) * SP + (e & 15)] = s1v[i];
        }
    }
    load_step(s_first, mrA, brA);
    if (s_first + 2 < nseg) load_step(s_first + 1, mrB, brB);
    __syncthreads();
    int cur = 0;
    // one step: S_start(s + 1) = M_s S_start(s) + B_s from the registers of slot (mr, br), which
    // then receive step s + 2 (in flight during the next step)
    auto step = [&](int64_t s, float4 (&mr)[TPW][NM], f32x4 (&br)[TPW]) __attribute__((always_inline)) {
        f32x4 acc[TPW];
#pragma unroll
        for (int q = 0; q < TPW; ++q) acc[q] = br[q];
        const float4 (&mc)[TPW][NM] = mr;
        // this lane's S_start(s) operands, all read from LDS before the products (one wait)
        const float* Sc = sS[cur];
        float sv[NM][4];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[m][e] = Sc[(16 * m + 4 * lc + e) * SP + li];
        wave_fence();
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sb = sv[m][e];
#pragma unroll
                for (int q = 0; q < TPW; ++q) {
                    const float4& a4 = mc[q][m];
                    const float av = e == 0 ? a4.x : e == 1 ? a4.y : e == 2 ? a4.z : a4.w;
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, sb, acc[q], 0, 0, 0);
                }
            }
        if (s + 3 < nseg) load_step(s + 2, mr, br);  // the slot's operands are consumed
        float* dst = sg.S + ((slot0 + s + 1) * H + h) * DK * DV + cb * 16;
        float* Sn = sS[cur ^ 1];
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
            const int r = wave + NWS * q;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * r + 4 * lc + v;
                Sn[row * SP + li] = acc[q][v];
                dst[static_cast<int64_t>(row) * DV + li] = acc[q][v];
            }
        }
        __syncthreads();                             // S_start(s + 1) complete in LDS
        cur ^= 1;
    };
    for (int64_t s = s_first; s + 1 < nseg; s += 2) {
        step(s, mrA, brA);
        if (s + 2 >= nseg) break;
        step(s + 1, mrB, brB);
    }
}

// ---- host side --------------------------------------------------------------------------------
int64_t slot_count(int32_t n_seqs, int64_t total_tokens, bool varlen, int32_t B, int64_t T, int tok) {
    if (!varlen) return static_cast<int64_t>(B) * ((T + tok - 1) / tok);
    return total_tokens / tok + n_seqs + 1;
}

size_t record_bytes(int32_t dk, bool precise) {
    if (dk == 128) return precise ? Rec<128, true>::BYTES : Rec<128, false>::BYTES;
    return precise ? Rec<64, true>::BYTES : Rec<64, false>::BYTES;
}

// Segments pay when the state pass would leave most of the chip idle -- few (sequence, head)
// column blocks -- and sequences are long on average.  A pure function of the sizes, so that
// the workspace query and the launch agree.
bool use_segments(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dv) {
    const int64_t wgs = static_cast<int64_t>(n_seqs) * H * (dv / 64);   // 64-column units
    return wgs <= 128 && total_tokens >= 2 * SEG_TOK * static_cast<int64_t>(n_seqs);
}
int64_t seg_slot_bound(int32_t n_seqs, int64_t total_tokens) {   // packed and fixed batches
    return total_tokens / SEG_TOK + n_seqs + 1;
}
size_t record_area(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dk, bool precise) {
    const int64_t slots = total_tokens / (precise ? 16 : 32) + n_seqs + 1;   // packed and fixed batches
    const size_t b = static_cast<size_t>(slots) * static_cast<size_t>(H) * record_bytes(dk, precise);
    return (b + 255) & ~static_cast<size_t>(255);
}

template <int DK, int IDT, int ODT, bool PRECISE, int NW, bool CKPT, int MODE>
void launch_state(const ChunkArgs& a, int64_t nslots, const uint8_t* ws, const SegArgs& sg,
                  int64_t units, int nvx, hipStream_t stream) {
    const int64_t groups = (units + 7) / 8;
    const int32_t n_vblk = a.dv / (16 * NW);
    hipLaunchKernelGGL((chunk_state_kernel<DK, IDT, ODT, PRECISE, NW, CKPT, MODE>),
                       dim3(static_cast<unsigned>(groups * 8 * nvx)), dim3(64 * (NW + state_helpers(NW))), 0,
                       stream, a, n_vblk, nslots, ws, sg);
}

template <int DK, int IDT, int ODT, bool PRECISE, int MODE, int NW = STATE_WAVES>
void launch_state_ck(const ChunkArgs& a, int64_t nslots, const uint8_t* ws, const SegArgs& sg,
                     int64_t units, int nvx, hipStream_t stream) {
    if (a.ckpt) launch_state<DK, IDT, ODT, PRECISE, NW, true, MODE>(a, nslots, ws, sg, units, nvx, stream);
    else launch_state<DK, IDT, ODT, PRECISE, NW, false, MODE>(a, nslots, ws, sg, units, nvx, stream);
}

// MI355X's last-level cache (Infinity Cache): 256 MB
constexpr int64_t LLC_BYTES = int64_t(256) << 20;

// A second stream per device for head-group concurrency, forked from and joined to the caller's
// stream by events (capturable: the side stream joins a capture through the fork event).  The
// mutex keeps each call's record-wait pairs together, so that no call waits on another's fork.
constexpr int SIDE_MAX_DEVICES = 64;
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[SIDE_MAX_DEVICES];

// fn(s0, s1) launches one part of the work on each stream.  Runs both parts on `stream` when the
// caller allows only its own stream, or when a capture is under way and the side stream does
// not exist yet (creating it then is not allowed).
template <typename F>
hipError_t on_two_streams(const ChunkArgs& a, hipStream_t stream, F&& fn) {
    if (a.single_stream) return fn(stream, stream);
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SIDE_MAX_DEVICES) return fn(stream, stream);
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream& sd = g_side[dev];
    if (sd.s == nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(stream, &cs)) != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone) return fn(stream, stream);
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        hipStream_t s = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        sd.s = s; sd.fork = f; sd.join = j;
    }
    if ((e = hipEventRecord(sd.fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(sd.s, sd.fork, 0)) != hipSuccess) return e;
    const hipError_t r = fn(stream, sd.s);
    // the join is recorded whatever fn returned: the caller's stream must not run ahead of work
    // already queued on the side stream
    if ((e = hipEventRecord(sd.join, sd.s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, sd.join, 0)) != hipSuccess) return e;
    return r;
}

// Segmented 16-bit prefills at d_k = d_v = 128 run as two head groups on two streams: the
// kernels of one group fill what the other's leave idle (a pass-1 chain beside intra-block
// streaming, a kernel's tail beside the next).  Measured on the packed 2^20-token, 8-head
// workload: 6.71 ms as one launch sequence, 6.39-6.48 ms as two concurrent halves.
bool split_heads(const ChunkArgs& a, bool segmented) {
    return segmented && a.in_dtype != KDA_F32 && a.dk == 128 && a.dv == 128 && a.heads == a.H &&
           a.H >= 2;
}

template <int DK, int IDT, int GDT, int ODT>
hipError_t launch_t(const ChunkArgs& a, hipStream_t stream) {
    constexpr bool PRECISE = (IDT == KDA_F32);
    const int64_t total = static_cast<int64_t>(a.B) * a.T;
    if (split_heads(a, use_segments(a.n_seqs, total, a.H, a.dv))) {
        ChunkArgs g0 = a, g1 = a;
        g0.heads = a.H / 2;
        g1.head0 = g0.heads;
        g1.heads = a.H - g0.heads;
        return on_two_streams(a, stream, [&](hipStream_t s0, hipStream_t s1) -> hipError_t {
            const hipError_t e = launch_t<DK, IDT, GDT, ODT>(g0, s0);
            if (e != hipSuccess) return e;
            return launch_t<DK, IDT, GDT, ODT>(g1, s1);
        });
    }
    const int64_t nslots = slot_count(a.n_seqs, total, a.cu != nullptr, a.B, a.T, Rec<DK, PRECISE>::TOK);
    uint8_t* ws = static_cast<uint8_t*>(a.workspace);
    const int64_t intra_wgs = nslots * a.heads;
    const bool segmented = use_segments(a.n_seqs, total, a.H, a.dv);
    if (intra_wgs > 0) {
        // 16-bit inputs: the token-per-lane kernel; fp32 inputs (split-bf16 records): the
        // split-operand kernel
        if constexpr (!PRECISE) {
            // Records that fit the last-level cache are stored with the default policy, so that
            // the passes after find them there; larger ones stream past it (measured: the
            // non-temporal hint costs 12% at 230 MB of records and saves 1.3% at 7.4 GB)
            const bool nt = nslots * a.H * Rec<DK, false>::BYTES > LLC_BYTES;
#define KDA_INTRA(G, N)                                                                        \
            hipLaunchKernelGGL((chunk_intra_tok_kernel<DK, GDT, G, N>),                       \
                               dim3(static_cast<unsigned>(intra_wgs)), dim3(64), 0, stream, a, nslots, ws)
            if (a.gate_A) { if (nt) KDA_INTRA(true, true); else KDA_INTRA(true, false); }
            else { if (nt) KDA_INTRA(false, true); else KDA_INTRA(false, false); }
#undef KDA_INTRA
        } else if (a.gate_A) {
            hipLaunchKernelGGL((chunk_intra_kernel<DK, IDT, GDT, PRECISE, true>),
                               dim3(static_cast<unsigned>(intra_wgs)), dim3(64), 0, stream, a, nslots, ws);
        } else {
            hipLaunchKernelGGL((chunk_intra_kernel<DK, IDT, GDT, PRECISE, false>),
                               dim3(static_cast<unsigned>(intra_wgs)), dim3(64), 0, stream, a, nslots, ws);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int32_t n_vblk = a.dv / (16 * STATE_WAVES);
    SegArgs sg{};
    if (!segmented) {
        launch_state_ck<DK, IDT, ODT, PRECISE, 0>(a, nslots, ws, sg, static_cast<int64_t>(a.n_seqs) * a.heads,
                                                  n_vblk, stream);
        return hipGetLastError();
    }
    // Long sequences: pass 1, the scan of segment pairs, pass 2.  With d_k = d_v = 128 the
    // segment passes use 8-wave workgroups: one covers all 128 columns of a state, M or B, so a
    // (segment, head) streams its records into two CUs instead of four.
    const size_t st = static_cast<size_t>(seg_slot_bound(a.n_seqs, total)) * a.H * DK;
    sg.S = reinterpret_cast<float*>(ws + record_area(a.n_seqs, total, a.H, DK, PRECISE));
    sg.B = sg.S + st * a.dv;
    sg.M = sg.B + st * a.dv;
    sg.seg_shift = SEG_SHIFT;
    sg.slots = a.cu ? seg_slot_bound(a.n_seqs, total)
                    : static_cast<int64_t>(a.B) * (a.T <= 0 ? 1 : (a.T + SEG_TOK - 1) / SEG_TOK);
    const int64_t seg_units = sg.slots * a.heads;
    constexpr int NW = SEG_WAVES;
    const bool wide = (DK == 128 && a.dv == 128);
    const int nw = wide ? 2 * NW : NW;
    sg.n_vblk_m = DK / (16 * nw);
    const int nvb = a.dv / (16 * nw);
    // 16-bit inputs at d_k = d_v = 128: pass 1 runs the pairs of every segment but the last, M
    // and B together (chunk_pair_kernel); the scan then starts from the initial state and pass 2
    // runs every segment.  Otherwise pass 1 runs segment 0 whole and the column blocks of the
    // middle segments' M and B apart.
    if constexpr (DK == 128 && !PRECISE) {
        if (wide) {
            sg.from0 = 1;
            if (seg_units > 0)
                hipLaunchKernelGGL((chunk_pair_kernel<IDT>), dim3(static_cast<unsigned>(seg_units)), dim3(512), 0,
                                   stream, a, nslots, ws, sg);
        }
    }
    if (!sg.from0) {
        if (wide)
            launch_state_ck<DK, IDT, ODT, PRECISE, 1, 2 * NW>(a, nslots, ws, sg, seg_units, sg.n_vblk_m + nvb, stream);
        else
            launch_state_ck<DK, IDT, ODT, PRECISE, 1, NW>(a, nslots, ws, sg, seg_units, sg.n_vblk_m + nvb, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((seg_scan_kernel<DK>),
                       dim3(static_cast<unsigned>((static_cast<int64_t>(a.n_seqs) * a.heads + 7) / 8 * 8 * (a.dv / 16))),
                       dim3(64 * scan_waves(DK)), 0, stream, a, sg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (wide)
        launch_state_ck<DK, IDT, ODT, PRECISE, 2, 2 * NW>(a, nslots, ws, sg, seg_units, nvb, stream);
    else
        launch_state_ck<DK, IDT, ODT, PRECISE, 2, NW>(a, nslots, ws, sg, seg_units, nvb, stream);
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

// Workspace: one record per (head, record slot: 32 tokens for 16-bit inputs, 16 for fp32);
// for segmented launches, then the segment start states, B and M per (segment slot, head).
size_t chunk_workspace_bytes(int32_t n_seqs, int64_t total_tokens, int32_t H, int32_t dk,
                             int32_t dv, int32_t in_dtype) {
    if (fused_eligible(in_dtype, dk, dv, n_seqs, H)) return 0;
    size_t b = record_area(n_seqs, total_tokens, H, dk, in_dtype == KDA_F32);
    if (use_segments(n_seqs, total_tokens, H, dv))
        b += static_cast<size_t>(seg_slot_bound(n_seqs, total_tokens)) * H * dk *
             (2 * static_cast<size_t>(dv) + dk) * 4;
    return b;
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream) {
    if (fused_eligible(a.in_dtype, a.dk, a.dv, a.n_seqs, a.H)) return launch_fused(a, stream);
    if (a.dk == 128) return dispatch<128>(a, stream);
    return dispatch<64>(a, stream);
}

}  // namespace kda
