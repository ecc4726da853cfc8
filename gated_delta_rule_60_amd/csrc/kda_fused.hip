// kda_fused.hip -- single-kernel chunked prefill for 16-bit inputs at d_k = d_v = 128.
//
// Pages (titles as published):
//   [bagrov] "Архитектура Kimi K3: как открытая модель с миллионным контекстом конкурирует с
//            лидерами рынка" (bagrov.by): § "Уровень чипа: специализированное ядро FlashKDA"
//            (the tokens of a block are processed together, then the state is passed on),
//            § "Уровень графического ускорителя: планировщик длинного контекста" (a long sequence
//            is cut into segments whose transitions are computed in parallel on one GPU and
//            combined exactly).
//   [habr]   "Как устроена Kimi K3: …" (savepearlharbor.com), § "Последовательность: три KDA на
//            один глобальный MLA" (the bound g >= -5 makes every 16-token block, diagonal ones
//            included, a dense product).
//
// One workgroup of twelve waves runs one (sequence, head) from its inputs to its outputs; the
// launch serves 16-bit inputs at d_k = d_v = 128 when the (sequence, head) units fill the chip.
// The block form is the one of the two-kernel path (kda_chunk.hip), and so is the 32-token record:
// two 16-token sub-blocks with -Kt = -e^G k, Qt = e^G q (scaled), Kb = e^{G_31 - G} k in fp16 MFMA
// fragment order (Kb^T of both sub-blocks joined per lane), T'_00, -C, T'_11, P_00, P_10, P_11 and
// the decay over the record.  Here the records never leave LDS.  In iteration r:
//   * four producer waves, one per 32-channel group, build record r + 2 from inputs loaded into
//     registers during the previous iteration: the gate, the cumsums, the factors, Kt / Qt / Kb
//     and their partial A, P and cross products over their 32 channels;
//   * consumer waves 0-2 finish record r + 1: they sum its partial products in a fixed order, form
//     T'_00 and T'_11 by forward substitution, and P_00, P_10, P_11 and -C = -Kt_1 Kb_0^T in fp16
//     (T'_10 = -T'_11 C T'_00 is applied below, so it is never formed);
//   * eight consumer waves, 16 state columns each, pass the fp32 state through record r:
//     X = V - Kt S, O = Qt S, W_0 = T'_00 X_0, W_1 = T'_11 (X_1 - C W_0), O += P W,
//     S <- Diag(e^{G_31}) S + Kb^T W, and store o.
// The V rows of record r + 1 stream into LDS by direct-to-LDS loads while record r is processed,
// so the kernel reads q, k, v, beta and g (or z) once and writes o once.  Tokens past a
// sequence's end read as zeros through the buffer ranges (identity records).
#include "kda_chunk_util.hpp"

namespace kda {
namespace {

constexpr int FDK = 128, FDV = 128;
constexpr int NPROD = 4;                 // producer waves (one per 32-channel group)
constexpr int NCONS = 8;                 // consumer waves (16 state columns each)
constexpr int NWAVE = NPROD + NCONS;
constexpr int RT = 32;                   // tokens per record
constexpr int FE2 = 16 * FDK * 2;        // bytes of one fp16 [16][128] record array
constexpr int F_OFF_T = 6 * FE2;         // T'_00, -C, T'_11 (fp16 [16][16] tiles, fragT)
constexpr int F_OFF_P = F_OFF_T + 1536;  // P_00, P_10, P_11
constexpr int F_OFF_G = F_OFF_P + 1536;  // e^{G_31} - 1 per channel, fp32
constexpr int F_REC = F_OFF_G + FDK * 4; // 28,160 bytes
constexpr int F_TILE = RT * FDK * 2;     // a bf16 [32][128] tile, 8 KiB

// LDS of one workgroup (149 KiB): three records (consumed, being finished, being built), two V
// tiles, two sets of the producers' partial products, the gate rates, beta of three records and
// the two diagonal A tiles of the record being finished.
struct __attribute__((aligned(16))) FusedLds {
    uint8_t rec[3][F_REC];
    f32x4 part[2][NPROD][6][64];         // A_0, A_1, P_0, P_1, C, Q in accumulator order
    float rate[2][FDK];                  // gate rates: hi, lo
    float beta[3][RT];
    float sA[2][16][16];                 // A_00, A_11 of the record being finished (fp32)
};

// V tiles: a 256-byte bf16 row holds 16 chunks of 16 bytes, chunk c stored at c ^ (row & 15), so
// the consumers' column reads spread over the banks.
__device__ __forceinline__ int t16_off(int r, int byte) {
    return r * 256 + ((((byte >> 4) ^ r) & 15) << 4) + (byte & 15);
}

// What one workgroup runs: a token range of one (sequence, head), where its state starts and
// ends, and whether it emits o (a segment's pair pass does not).
struct FUnit {
    int64_t tok0;        // first token (row of the [tokens, H, .] layout, before the head)
    int64_t ntok;        // tokens in the range
    int64_t seq_off;     // offset of tok0 within its sequence (checkpoint positions)
    int64_t ck_base;     // checkpoint slot base of the sequence
    const float* init;   // initial state, nullptr: zeros
    float* fin;          // final state, nullptr: not stored
    int h;
};

struct FCtx {
    const ChunkArgs* p;
    int64_t H, nrec;
    uint32_t rowb, rowg;
    int wave, lane, h;
};

__device__ __forceinline__ int rec_tokens(const FUnit& u, int64_t r) {
    const int64_t rem = u.ntok - RT * r;
    return static_cast<int>(rem < 0 ? 0 : rem < RT ? rem : RT);
}

// ---- producer inputs: one record's k, q, g or z for the lane's channels, in registers -------
// Lane (m, q) of producer kk owns token m of each sub-block and channels 32 kk + 16 (j >> 2) +
// 4 q + (j & 3), j = 0..7 -- the channels its 16-byte unit of a frag32 record array holds.  Wave
// 0 also holds beta of token `lane`.  Loaded two records ahead of use; rows past the range read 0.
template <int GSZ>
struct PIn {
    uint32_t k[2][4], q[2][4], g[2][2 * GSZ];
    uint16_t beta;                        // bf16 bits
};
template <int GSZ>
__device__ __forceinline__ void load_inputs(const FCtx& c, const FUnit& u, int64_t r, PIn<GSZ>& in) {
    const ChunkArgs& p = *c.p;
    const int m = c.lane & 15, q = c.lane >> 4, kk = c.wave;
    const int nt = rec_tokens(u, r);
    const int64_t row0 = (u.tok0 + RT * r) * c.H + c.h;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc_u(static_cast<const uint16_t*>(p.k) + row0 * FDK, nt * c.rowb);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc_u(static_cast<const uint16_t*>(p.q) + row0 * FDK, nt * c.rowb);
    const __amdgpu_buffer_rsrc_t gr = make_rsrc_u(static_cast<const uint8_t*>(p.g) + row0 * FDK * GSZ, nt * c.rowg);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int tok = 16 * s + m, ch = 32 * kk + 16 * hh + 4 * q;
            const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(kr, tok * c.rowb + 2 * ch, 0, 0);
            in.k[s][2 * hh] = a[0]; in.k[s][2 * hh + 1] = a[1];
            const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(qr, tok * c.rowb + 2 * ch, 0, 0);
            in.q[s][2 * hh] = b[0]; in.q[s][2 * hh + 1] = b[1];
            if constexpr (GSZ == 4) {
                const u32x4 g4 = __builtin_amdgcn_raw_buffer_load_b128(gr, tok * c.rowg + 4 * ch, 0, 0);
                in.g[s][4 * hh] = g4[0]; in.g[s][4 * hh + 1] = g4[1]; in.g[s][4 * hh + 2] = g4[2]; in.g[s][4 * hh + 3] = g4[3];
            } else {
                const u32x2 g2 = __builtin_amdgcn_raw_buffer_load_b64(gr, tok * c.rowg + 2 * ch, 0, 0);
                in.g[s][2 * hh] = g2[0]; in.g[s][2 * hh + 1] = g2[1];
            }
        }
    if (kk == 0)
        in.beta = __builtin_amdgcn_raw_buffer_load_b16(
            make_rsrc_u(static_cast<const uint16_t*>(p.beta) + row0, nt * static_cast<uint32_t>(c.H) * 2),
            c.lane * static_cast<uint32_t>(c.H) * 2, 0, 0);
}

// ---- producer: one record over one 32-channel group ---------------------------------------
// The gate, the cumsums (DPP scans across the 16 lanes of a row), the factors, Kt / Qt / Kb and
// e^{G_31} - 1 into the record, and the partial A, P (fp32 MFMAs) and cross products C = Kt_1
// Kb_0^T, Q = Qt_1 Kb_0^T (fp16 MFMAs) over the group's channels into `part`.
template <int GDT, bool GATE>
__device__ __forceinline__ void produce(const ChunkArgs& p, const PIn<(GDT == KDA_F32) ? 4 : 2>& in,
                                        uint8_t* rec, f32x4 (*part)[64], float* beta,
                                        const float (*rate)[FDK], int nt, int kk, int lane) {
    constexpr float LOG2E = 1.4426950408889634f;
    asm volatile("" : "+v"(lane));       // as in finish(): no lane-derived values held across records
    const int m = lane & 15, q = lane >> 4;
    if (kk == 0 && lane < RT) beta[lane] = bf16_val(in.beta);
    auto raw16 = [](const uint32_t* w, int j) -> float {      // element j of packed bf16 words
        return (j & 1) ? __uint_as_float(w[j >> 1] & 0xffff0000u) : __uint_as_float(w[j >> 1] << 16);
    };
    float4 rt4[2][2];                    // [hi, lo][channel half]
    if constexpr (GATE) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            rt4[w][0] = *reinterpret_cast<const float4_ma*>(&rate[w][32 * kk + 4 * q]);
            rt4[w][1] = *reinterpret_cast<const float4_ma*>(&rate[w][32 * kk + 16 + 4 * q]);
        }
    }
    const bool full = (nt == RT);
    const float keep[2] = {m < nt ? 1.f : 0.f, 16 + m < nt ? 1.f : 0.f};
    float x[2][8], e1[2][8], gm[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float gv;
            if constexpr (GATE) {
                const float z = (GDT == KDA_F32) ? __uint_as_float(in.g[s][j]) : raw16(in.g[s], j);
                auto pick = [&](const float4& r4) {
                    return (j & 3) == 0 ? r4.x : (j & 3) == 1 ? r4.y : (j & 3) == 2 ? r4.z : r4.w;
                };
                gv = gate_log_decay(pick(rt4[0][j >> 2]), pick(rt4[1][j >> 2]), z, p.g_min);
                if (!full) gv *= keep[s];                        // 0 past the record's tokens
            } else if constexpr (GDT == KDA_F32) {
                gv = __uint_as_float(in.g[s][j]);
            } else {
                gv = raw16(in.g[s], j);
            }
            x[s][j] = gv * LOG2E;
        }
    // inclusive cumsum over the 16 tokens of each row and sub-block (log2 units)
#define KDA_SCAN_STEP(CTRL)                                                                          \
    _Pragma("unroll") for (int s = 0; s < 2; ++s)                                                  \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                                  \
        x[s][j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[s][j]), CTRL, 0xf, 0xf, true));
    KDA_SCAN_STEP(0x111)
    KDA_SCAN_STEP(0x112)
    KDA_SCAN_STEP(0x114)
    KDA_SCAN_STEP(0x118)
#undef KDA_SCAN_STEP
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) e1[s][j] = fexp2(x[s][j]);             // e^{G} <= 1
    // e^{G_15}: lane 15 of the row (bitmask swizzle: lane -> (lane & 16) | 15)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            gm[s][j] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(e1[s][j]), 0x1F0));
    const bool unit_scale = (p.scale == 1.f);

    f32x4 accA[2] = {zero4(), zero4()}, accP[2] = {zero4(), zero4()}, accC = zero4(), accQ = zero4();
    // sub-block 0: Kt, Qt, Kd with its own cumsum; Kb_0 = Kd e^{G_15} <= 1 kept for the cross products
    float kb0[8];
    {
        float kt[8], qt[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float kv = raw16(in.k[0], j);
            kt[j] = kv * e1[0][j];
            const float kd = kv * fexp2(-x[0][j]);                       // e^{-G} <= e^80
            accA[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[j], kd, accA[0], 0, 0, 0);
            // the output scale rides on Qt and P
            qt[j] = raw16(in.q[0], j) * (unit_scale ? e1[0][j] : e1[0][j] * p.scale);
            accP[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt[j], kd, accP[0], 0, 0, 0);
            kb0[j] = kd * gm[0][j];
        }
        // Kt is stored negated: the state step forms V - Kt S as one product onto V
        *reinterpret_cast<uint4*>(rec + (64 * kk + lane) * 16) =
            make_uint4(f16_pair(-kt[0], -kt[1]), f16_pair(-kt[2], -kt[3]), f16_pair(-kt[4], -kt[5]), f16_pair(-kt[6], -kt[7]));
        *reinterpret_cast<uint4*>(rec + FE2 + (64 * kk + lane) * 16) =
            make_uint4(f16_pair(qt[0], qt[1]), f16_pair(qt[2], qt[3]), f16_pair(qt[4], qt[5]), f16_pair(qt[6], qt[7]));
    }
    // sub-block 1: the same with its own cumsum, plus C = Kt_1 Kb_0^T and Q = Qt_1 Kb_0^T; the
    // record holds Kt_1, Qt_1 scaled from the record's first token
    {
        float kt[8], qt[8], kb1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float kv = raw16(in.k[1], j);
            kt[j] = kv * e1[1][j];
            const float kd = kv * fexp2(-x[1][j]);
            accA[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[j], kd, accA[1], 0, 0, 0);
            qt[j] = raw16(in.q[1], j) * (unit_scale ? e1[1][j] : e1[1][j] * p.scale);
            accP[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt[j], kd, accP[1], 0, 0, 0);
            kb1[j] = kd * gm[1][j];
        }
        f16x8 k1h, b0h, q1h;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            k1h[j] = static_cast<_Float16>(kt[j]);
            b0h[j] = static_cast<_Float16>(kb0[j]);
            q1h[j] = static_cast<_Float16>(qt[j]);
        }
        accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1h, b0h, accC, 0, 0, 0);
        accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(q1h, b0h, accQ, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            kt[j] *= gm[0][j];
            qt[j] *= gm[0][j];
        }
        *reinterpret_cast<uint4*>(rec + 3 * FE2 + (64 * kk + lane) * 16) =
            make_uint4(f16_pair(-kt[0], -kt[1]), f16_pair(-kt[2], -kt[3]), f16_pair(-kt[4], -kt[5]), f16_pair(-kt[6], -kt[7]));
        *reinterpret_cast<uint4*>(rec + 4 * FE2 + (64 * kk + lane) * 16) =
            make_uint4(f16_pair(qt[0], qt[1]), f16_pair(qt[2], qt[3]), f16_pair(qt[4], qt[5]), f16_pair(qt[6], qt[7]));
        // Kb^T of both sub-blocks in fragKb order: Kb_0 scaled to the record's last token
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 32 * kk + 16 * (j >> 2) + 4 * q + (j & 3);
            uint16_t* const kt16 = reinterpret_cast<uint16_t*>(rec + kb_tile_off(c >> 4, 8, 2 * FE2, 5 * FE2));
            kt16[fragkb(c, 0, m)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(kb0[j] * gm[1][j]));
            kt16[fragkb(c, 1, m)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(kb1[j]));
        }
    }
    if (m == 15) {   // e^{G_31} - 1 per channel: the product of the sub-blocks' e^{G_15}
        float* gp = reinterpret_cast<float*>(rec + F_OFF_G) + 32 * kk + 4 * q;
        float d[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] = fmaf(gm[0][j], gm[1][j], -1.f);
        *reinterpret_cast<float4*>(gp) = make_float4(d[0], d[1], d[2], d[3]);
        *reinterpret_cast<float4*>(gp + 16) = make_float4(d[4], d[5], d[6], d[7]);
    }
    part[0][lane] = accA[0];
    part[1][lane] = accA[1];
    part[2][lane] = accP[0];
    part[3][lane] = accP[1];
    part[4][lane] = accC;
    part[5][lane] = accQ;
}

// ---- consumer waves 0-2: finish a record from the four partial products --------------------
// The sums run in a fixed order (deterministic).  Wave 0: A_ss = beta * strict_lower(sum) of both
// sub-blocks into LDS, then T'_ss = (I + A_ss)^{-1} Diag(beta) by forward substitution, row by
// row: lanes (s, j, h) = (lane >> 5, (lane >> 1) & 15, lane & 1) hold rows k = 2 i + h of column j
// of sub-block s, each row's dot product split over the lane pair h = 0, 1 and summed across it
// with one DPP add.  Wave 1: P_00, P_11 (lower, the diagonal included).  Wave 2: -C and P_10 = Q.
__device__ __forceinline__ void finish(const f32x4 (*part)[6][64], const float* beta, uint8_t* rec,
                                       float (*sA)[16][16], int pw, int lane) {
    // an opaque copy of the lane index: the masks below are formed per record instead of being
    // hoisted out of the record loop and held in registers across it
    asm volatile("" : "+v"(lane));
    const int m = lane & 15, q = lane >> 4;
    auto sum4 = [&](int tile) -> f32x4 {
        return ((part[0][tile][lane] + part[1][tile][lane]) + part[2][tile][lane]) + part[3][tile][lane];
    };
    uint16_t* const tT = reinterpret_cast<uint16_t*>(rec + F_OFF_T);
    uint16_t* const tP = reinterpret_cast<uint16_t*>(rec + F_OFF_P);
    if (pw == 0) {
        // A(r, c) of sub-block s at sA[s][r][8 (c & 1) + (c >> 1)]: a lane reads its half of a row
        // (the columns of one parity) as two float4
        const int mc = 8 * (m & 1) + (m >> 1);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const f32x4 a = sum4(sb);                   // lane (m, q): rows 4 q + i, column m
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q + i;
                sA[sb][r][mc] = (m < r) ? a[i] * beta[16 * sb + r] : 0.f;
            }
        }
        wave_fence();   // A is read across lanes below
        const int sb = lane >> 5, jc = (lane >> 1) & 15, h = lane & 1;
        const float (*const A)[16] = sA[sb];
        // tk[i] = T(2 i + h, jc).  Rows in blocks of four: the block's dot products over the rows
        // already formed (each lane over its parity, summed across the pair with one DPP add),
        // then the block's own 4 x 4 lower triangle row by row, in both lanes of the pair alike.
        float tk[8];
        auto half4 = [&](int r, int u) -> float4 { return *reinterpret_cast<const float4_ma*>(&A[r][8 * h + 4 * u]); };
        auto pair_sum = [](float x) -> float {   // x + the partner lane's x (quad_perm [1, 0, 3, 2])
            return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
        };
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            // A(4I + a, 4I + b) for b < a: the two float2 at parity offsets 2I (even b) and 8 + 2I (odd b)
            float2 ev[4], od[4];
#pragma unroll
            for (int a4 = 1; a4 < 4; ++a4) {
                ev[a4] = *reinterpret_cast<const float2*>(&A[4 * I + a4][2 * I]);
                od[a4] = *reinterpret_cast<const float2*>(&A[4 * I + a4][8 + 2 * I]);
            }
            float c[4];
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int r = 4 * I + a4;
                float acc[2] = {0.f, 0.f};
#pragma unroll
                for (int u = 0; u < (2 * I + 3) / 4; ++u) {
                    const float4 v = half4(r, u);
                    const float av[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * u + e < 2 * I) acc[e & 1] = fmaf(av[e], tk[4 * u + e], acc[e & 1]);
                }
                const float dot = (I == 0) ? 0.f : pair_sum(acc[0] + acc[1]);
                c[a4] = ((r == jc) ? 1.f : 0.f) - dot;
            }
            const float t0 = c[0];
            const float t1 = fmaf(-ev[1].x, t0, c[1]);
            const float t2 = fmaf(-od[2].x, t1, fmaf(-ev[2].x, t0, c[2]));
            const float t3 = fmaf(-ev[3].y, t2, fmaf(-od[3].x, t1, fmaf(-ev[3].x, t0, c[3])));
            tk[2 * I] = h ? t1 : t0;
            tk[2 * I + 1] = h ? t3 : t2;
        }
        const float bj = beta[16 * sb + jc];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            tT[512 * sb + fragT(2 * i + h, jc)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(tk[i] * bj));
    } else if (pw == 1) {
        const f32x4 p0 = sum4(2), p1 = sum4(3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * q + i;
            tP[fragT(r, m)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>((m <= r) ? p0[i] : 0.f));
            tP[512 + fragT(r, m)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>((m <= r) ? p1[i] : 0.f));
        }
    } else if (pw == 2) {
        const f32x4 c = sum4(4), qq = sum4(5);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tT[256 + fragT(4 * q + i, m)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-c[i]));
            tP[256 + fragT(4 * q + i, m)] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(qq[i]));
        }
    }
}

// ---- the two roles' loops --------------------------------------------------------------------
// Record x is built by the producers in iteration x - 2, finished by consumer waves 0-2 in
// iteration x - 1 and consumed in iteration x, all out of LDS slot x % 3 (partial products x % 2,
// beta x % 3).  The producers' inputs arrive in registers, loaded one iteration before their use.
// Both loops issue the same workgroup barriers: three in the prologue (gate rates, record 0
// built, record 0 finished and record 1 built) and one per record.
template <int GDT, bool GATE>
__device__ __forceinline__ void producer_loop(const FCtx& c, const FUnit& u, FusedLds& L) {
    constexpr int GSZ = (GDT == KDA_F32) ? 4 : 2;
    const ChunkArgs& p = *c.p;
    const int wave = c.wave, lane = c.lane;
    const int nrec = static_cast<int>(c.nrec);
    PIn<GSZ> in;
    if constexpr (GATE) {
        if (wave < 2) {
            const GateRate gr = gate_rate(p.gate_A[static_cast<int64_t>(c.h) * FDK + 64 * wave + lane]);
            L.rate[0][64 * wave + lane] = gr.hi;
            L.rate[1][64 * wave + lane] = gr.lo;
        }
    }
    if (nrec > 0) load_inputs<GSZ>(c, u, 0, in);
    __syncthreads();
    if (nrec > 0) {
        produce<GDT, GATE>(p, in, L.rec[0], L.part[0][wave], L.beta[0], L.rate, rec_tokens(u, 0), wave, lane);
        if (nrec > 1) load_inputs<GSZ>(c, u, 1, in);
    }
    __syncthreads();
    if (nrec > 1) {
        produce<GDT, GATE>(p, in, L.rec[1], L.part[1][wave], L.beta[1], L.rate, rec_tokens(u, 1), wave, lane);
        if (nrec > 2) load_inputs<GSZ>(c, u, 2, in);
    }
    __syncthreads();
    // iteration r: build record r + 2 (inputs loaded during iteration r - 1), then load record r + 3
    for (int r = 0; r < nrec; ++r) {
        const int x = r + 2;
        if (x < nrec) {
            produce<GDT, GATE>(p, in, L.rec[x % 3], L.part[x & 1][wave], L.beta[x % 3], L.rate,
                               rec_tokens(u, x), wave, lane);
            if (x + 1 < nrec) load_inputs<GSZ>(c, u, x + 1, in);
        }
        __syncthreads();
    }
}

// Each consumer wave owns 16 state columns of the fp32 state for the whole range and emits o.
template <int GDT, bool GATE>
__device__ __forceinline__ void consumer_loop(const FCtx& c, const FUnit& u, FusedLds& L, uint8_t* V0, uint8_t* V1) {
    constexpr int O_STORES = 8;                        // o stores per lane and record
    const ChunkArgs& p = *c.p;
    const int lane = c.lane, ln = lane & 15, lq = lane >> 4;
    const int cw = c.wave - NPROD;
    const int64_t H = c.H;
    const int nrec = static_cast<int>(c.nrec);
    const int h = c.h;
    const int32_t vstride = static_cast<int32_t>(H) * FDV;
    const int col = 16 * cw + ln;                      // this lane's state column
    const bool o32 = (p.o_dtype == KDA_F32);
    const int osz = o32 ? 4 : 2;
    // the lane's rows of a record's V tile and o rows: tokens 4 lq + i (sub-block 0), 16 + ...
    int voff[8], ooff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int tok = (i < 4) ? 4 * lq + i : 16 + 4 * lq + (i - 4);
        voff[i] = t16_off(tok, 2 * col);
        ooff[i] = (tok * vstride + col) * osz;
    }

    // lane (ln, lq) holds S[16 i + 4 lq + rr][col] in S[i][rr]; an absent initial state is an
    // empty range, whose loads read 0
    f32x4 S[8];
    {
        const __amdgpu_buffer_rsrc_t ir = make_rsrc(u.init, u.init ? static_cast<uint32_t>(FDK * FDV * 4) : 0u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                S[i][rr] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    ir, ((16 * i + 4 * lq + rr) * FDV + col) * 4, 0, 0));
    }
    // V rows of record r into a [32][128] tile, one 1 KiB instruction per consumer wave
    auto issue_v = [&](int64_t r, uint8_t* tile) {
        const int nt = rec_tokens(u, r);
        const int64_t row0 = (u.tok0 + RT * r) * H + h;
        const __amdgpu_buffer_rsrc_t vr = make_rsrc_u(static_cast<const uint16_t*>(p.v) + row0 * FDV, nt * c.rowb);
        const int S_ = 64 * cw + lane, rr = S_ >> 4, ch = (S_ & 15) ^ (rr & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(tile + 1024 * cw),
                                                 16, rr * c.rowb + 16 * ch, 0, 0, CP_NT);
    };
    if (nrec > 0) issue_v(0, V0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();   // gate rates
    __syncthreads();   // record 0 built
    if (nrec > 0 && cw < 3) {
        __builtin_amdgcn_s_setprio(3);
        finish(L.part[0], L.beta[0], L.rec[0], L.sA, cw, lane);
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();   // record 0 finished, record 1 built
    // one record: vt holds its V rows, vnext receives those of the next record.  The two V tiles
    // are separate LDS arrays and the loop below alternates them in unrolled pairs, so the
    // compiler can tell the reads of vt from the transfer into vnext and does not wait for it.
    auto step = [&](int r, const uint8_t* vt, uint8_t* vnext) __attribute__((always_inline)) {
        // waves 0-2 first finish record r + 1 (built by the producers in the previous iteration),
        // before this record's transfers are issued, so their LDS accesses wait for none of them.
        // The finish is the longest dependent chain of a record, so these waves take the issue
        // arbitration of their SIMD while they run it.
        if (r + 1 < nrec && cw < 3) {
            __builtin_amdgcn_s_setprio(3);
            finish(L.part[(r + 1) & 1], L.beta[(r + 1) % 3], L.rec[(r + 1) % 3], L.sA, cw, lane);
            __builtin_amdgcn_s_setprio(0);
        }
        if (r + 1 < nrec) issue_v(r + 1, vnext);
        const uint8_t* rc = L.rec[r % 3];
        // X_s = V_s - Kt_s S (the record holds -Kt: one product accumulated onto V; the beta
        // scaling sits in T') and O_s = Qt_s S, contracting over d_k with S packed as the B operand
        f32x4 Y[2], O[2] = {zero4(), zero4()};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Y[0][i] = bf16_val(*reinterpret_cast<const uint16_t*>(vt + voff[i]));
            Y[1][i] = bf16_val(*reinterpret_cast<const uint16_t*>(vt + voff[4 + i]));
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const f16x8 ka0 = *reinterpret_cast<const f16x8*>(rc + 1024 * kk + 16 * lane);
            const f16x8 ka1 = *reinterpret_cast<const f16x8*>(rc + 3 * FE2 + 1024 * kk + 16 * lane);
            const f16x8 qa0 = *reinterpret_cast<const f16x8*>(rc + FE2 + 1024 * kk + 16 * lane);
            const f16x8 qa1 = *reinterpret_cast<const f16x8*>(rc + 4 * FE2 + 1024 * kk + 16 * lane);
            f16x8 sb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sb[i] = static_cast<_Float16>(S[2 * kk][i]);
                sb[4 + i] = static_cast<_Float16>(S[2 * kk + 1][i]);
            }
            Y[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka0, sb, Y[0], 0, 0, 0);
            Y[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka1, sb, Y[1], 0, 0, 0);
            O[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa0, sb, O[0], 0, 0, 0);
            O[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa1, sb, O[1], 0, 0, 0);
        }
        // W_0 = T'_00 X_0; X_1' = X_1 - C W_0; W_1 = T'_11 X_1'
        const f16x4 t00 = *reinterpret_cast<const f16x4*>(rc + F_OFF_T + 8 * lane);
        const f16x4 ncm = *reinterpret_cast<const f16x4*>(rc + F_OFF_T + 512 + 8 * lane);
        const f16x4 t11 = *reinterpret_cast<const f16x4*>(rc + F_OFF_T + 1024 + 8 * lane);
        const f32x4 X0 = Y[0], X1 = Y[1];
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
        {
            // O += P W (P and Qt carry the output scale); o rows of this record, stored with the
            // default cache policy so that the waves' partial lines merge in L2.  O_1 += [P_10 P_11]
            // [W_0; W_1] is one K = 32 product: a lane's k slots pair its W_0 and W_1 rows with the
            // same columns of P_10 and P_11.
            const f16x4 p00 = *reinterpret_cast<const f16x4*>(rc + F_OFF_P + 8 * lane);
            const f16x8 p1x = __builtin_shufflevector(*reinterpret_cast<const f16x4*>(rc + F_OFF_P + 512 + 8 * lane),
                                                      *reinterpret_cast<const f16x4*>(rc + F_OFF_P + 1024 + 8 * lane),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
            const int nt = rec_tokens(u, r);
            const __amdgpu_buffer_rsrc_t orr = make_rsrc_u(
                static_cast<char*>(p.o) + ((u.tok0 + RT * r) * H + h) * FDV * osz,
                static_cast<uint32_t>(nt * vstride * osz));
            const f32x4 O0 = __builtin_amdgcn_mfma_f32_16x16x16f16(p00, w0, O[0], 0, 0, 0);
            const f32x4 O1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(p1x, wx, O[1], 0, 0, 0);
            if (o32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O0[i]), orr, ooff[i], 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O1[i]), orr, ooff[4 + i], 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(O0[i]), orr, ooff[i], 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(O1[i]), orr, ooff[4 + i], 0, 0);
                }
            }
        }
        // S <- Diag(e^{G_31}) S + Kb^T W = S + Diag(e^{G_31} - 1) S + [Kb_0^T Kb_1^T] [W_0; W_1]
        const float* gam = reinterpret_cast<const float*>(rc + F_OFF_G);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * i + 4 * lq);
            const f16x8 ka = *reinterpret_cast<const f16x8*>(rc + kb_tile_off(i, 8, 2 * FE2, 5 * FE2) + 16 * lane);
            f32x4 acc;
            acc[0] = fmaf(S[i][0], gm.x, S[i][0]); acc[1] = fmaf(S[i][1], gm.y, S[i][1]);
            acc[2] = fmaf(S[i][2], gm.z, S[i][2]); acc[3] = fmaf(S[i][3], gm.w, S[i][3]);
            S[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, wx, acc, 0, 0, 0);
        }
        // checkpoint: the state after every ckpt_every tokens of the sequence
        if (p.ckpt) {
            const int64_t done = u.seq_off + RT * (r + 1);
            if (RT * (r + 1) <= u.ntok && done % p.ckpt_every == 0) {
                const int64_t slot = u.ck_base + done / p.ckpt_every - 1;
                if (slot < p.ckpt_slots) {
                    // the lane's offset from an opaque lane copy, formed here rather than held in
                    // registers across the record loop; the rows' offsets ride in soffset
                    int ln_ = lane;
                    asm volatile("" : "+v"(ln_));
                    const uint32_t vb = static_cast<uint32_t>((4 * (ln_ >> 4) * FDV + 16 * cw + (ln_ & 15)) * 4);
                    const __amdgpu_buffer_rsrc_t cr = make_rsrc_u(p.ckpt + (slot * H + h) * FDK * FDV, FDK * FDV * 4);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[i][rr]), cr, vb, (16 * i + rr) * FDV * 4, 0);
                }
            }
        }
        // V of the next record has landed (this record's o stores and a checkpoint may stay in flight)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(O_STORES));
        __syncthreads();
    };
    for (int r = 0; r < nrec; r += 2) {
        step(r, V0, V1);
        if (r + 1 < nrec) step(r + 1, V1, V0);
    }
    // the state the workgroup ends with
    if (u.fin) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                u.fin[static_cast<int64_t>(16 * i + 4 * lq + rr) * FDV + col] = S[i][rr];
    }
}

template <int GDT, bool GATE>
__global__ void __launch_bounds__(NWAVE * 64, 1) fused_kernel(ChunkArgs p) {
    constexpr int GSZ = (GDT == KDA_F32) ? 4 : 2;
    __shared__ FusedLds L;
    __shared__ __attribute__((aligned(16))) uint8_t V0[F_TILE], V1[F_TILE];   // V tiles of alternate records
    const int64_t H = p.H;
    const int h = static_cast<int>(blockIdx.x % H);
    const int n = static_cast<int>(blockIdx.x / H);
    if (n >= p.n_seqs) return;
    FUnit u{};
    u.h = h;
    int64_t bos, len;
    if (p.cu) {
        int64_t end;
        seq_bounds(p, n, bos, end);
        len = end - bos;
    } else {
        bos = static_cast<int64_t>(n) * p.T;
        len = p.T;
    }
    const int64_t useq = static_cast<int64_t>(n) * H + h;
    u.tok0 = bos;
    u.ntok = len;
    u.seq_off = 0;
    u.init = p.h0 ? p.h0 + useq * FDK * FDV : nullptr;
    u.fin = p.hT ? p.hT + useq * FDK * FDV : nullptr;
    u.ck_base = p.ckpt == nullptr ? 0
              : p.cu ? bos / p.ckpt_every + n : static_cast<int64_t>(n) * (p.T / p.ckpt_every);
    FCtx c;
    c.p = &p;
    c.H = H;
    c.nrec = (u.ntok + RT - 1) / RT;
    c.rowb = static_cast<uint32_t>(H * FDK * 2);
    c.rowg = static_cast<uint32_t>(H * FDK * GSZ);
    c.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    c.lane = threadIdx.x & 63;
    c.h = h;
    if (c.wave < NPROD) producer_loop<GDT, GATE>(c, u, L);
    else consumer_loop<GDT, GATE>(c, u, L, V0, V1);
}

template <int GDT, bool GATE>
hipError_t launch_t(const ChunkArgs& a, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(a.n_seqs) * a.H;
    if (units <= 0) return hipSuccess;
    hipLaunchKernelGGL((fused_kernel<GDT, GATE>), dim3(static_cast<unsigned>(units)), dim3(NWAVE * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Whole sequences in one launch when the (sequence, head) units fill the chip: one workgroup per
// CU.  With fewer units the two-kernel path serves: its state pass splits a state's columns over
// workgroups, or cuts long sequences into segments, where building every record in the workgroup
// that consumes it would be repeated across the segment passes.
bool fused_eligible(int32_t in_dtype, int32_t dk, int32_t dv, int32_t n_seqs, int32_t H) {
    return in_dtype == KDA_BF16 && dk == FDK && dv == FDV && static_cast<int64_t>(n_seqs) * H >= 256;
}

hipError_t launch_fused(const ChunkArgs& a, hipStream_t stream) {
    if (a.gate_A) {
        if (a.g_dtype == KDA_F32) return launch_t<KDA_F32, true>(a, stream);
        return launch_t<KDA_BF16, true>(a, stream);
    }
    if (a.g_dtype == KDA_F32) return launch_t<KDA_F32, false>(a, stream);
    return launch_t<KDA_BF16, false>(a, stream);
}

}  // namespace kda
