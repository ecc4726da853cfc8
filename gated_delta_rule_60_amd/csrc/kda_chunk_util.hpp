// kda_chunk_util.hpp -- device helpers shared by the chunked-prefill kernels (gfx950 only):
// vector types, buffer resources, MFMA operand layouts, sequence and segment bookkeeping.
#pragma once

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// s_waitcnt immediate for "vmcnt <= n", other counters unconstrained.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Buffer resource over [base, base + bytes): raw (unswizzled, stride 0) accesses whose byte offset
// lies outside the range read 0 and write nothing, so loads and stores need no branches and the
// compiler can count outstanding memory operations exactly.  Word 3 selects 32-bit data format.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_ma __attribute__((ext_vector_type(4), may_alias));   // 16-byte LDS units
constexpr int CP_NT = 2;   // buffer cache policy: non-temporal (data used once)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}
// The same for a base and size that are equal in every lane but that the compiler cannot prove
// uniform: taken from the first lane, so the descriptor stays in scalar registers and a load
// through it needs no loop over distinct lane values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b)));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
    return make_rsrc(reinterpret_cast<const void*>((hi << 32) | lo),
                     static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bytes))));
}

// 2^x with one v_exp_f32.  Every factor formed here lies in [2^-116, 2^116] (a 16-token span
// decays by at most e^-80), so the instruction's denormal flush never applies.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two fp32 values -> packed bf16 hi word and packed bf16 lo word (x = hi + lo to ~16 bits).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
    const float r0 = x0 - __uint_as_float(hi << 16);
    const float r1 = x1 - __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}
// Staged tiles are written as 16-bit (or fp32) elements and read back as whole 16-byte units
// through may_alias types, which makes these type-punned reads well defined.
typedef uint4 __attribute__((may_alias)) uint4_ma;
typedef float4 __attribute__((may_alias)) float4_ma;
__device__ __forceinline__ uint32_t f16_pair(float x0, float x1) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, f16x2));
}
__device__ __forceinline__ void split4(const f32x4& x, s16x4& hi, s16x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t h = bf16_bits(x[i]);
        hi[i] = static_cast<short>(h);
        lo[i] = static_cast<short>(bf16_bits(x[i] - bf16_val(h)));
    }
}
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 hb = static_cast<__bf16>(x[i]);
        hi[i] = hb;
        lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hb));
    }
}

// ---- layouts ---------------------------------------------------------------------------------
// [16][DK] 16-bit arrays (token-major): 16-byte units of 8 channels, unit index XOR (row & 7)
// so that the 16 rows of an MFMA fragment read fall in different banks.
template <int DK>
__device__ __forceinline__ int tok_major(int r, int c) {
    return r * DK + ((((c >> 3) ^ (r & 7))) << 3) + (c & 7);
}
// Record arrays are stored in MFMA fragment order, so that the state pass reads each operand
// with one contiguous 16- or 8-byte load per lane (1 KB / 512 B per wave, no bank conflicts):
//   frag32: [16][DK] operand of a 16x16x32 product (row = token, K = channel): fragment kk,
//           lane (m, q) holds channels 32kk + 4q + {0..3} in slots 0..3 and 32kk + 16 + 4q + {0..3}
//           in slots 4..7 -- the K order in which the state tiles are packed as the B operand.
//   frag16: [DK][16] operand of a 16x16x16 product (row = channel, K = token): tile i, lane
//           (m, q) holds channel 16i + m, tokens 4q .. 4q + 3.
//   fragKb: [DK][32] operand of a 16x16x32 product (row = channel, K = the 32 tokens of a
//           record): in tile i (1 KB), lane (m, q) holds channel 16i + m, tokens 4q .. 4q + 3 of
//           sub-block 0 in slots 0..3 and the same tokens of sub-block 1 in slots 4..7 -- the K
//           order in which W_0 and W_1 are joined as the B operand.  fragkb gives the half index
//           inside the tile; kb_tile_off the tile's byte offset in a record.
//   fragT : [16][16] operand of a 16x16x16 product: lane (m, q) holds row m, columns 4q .. 4q + 3.
__device__ __forceinline__ int frag32(int r, int c) {
    return ((c >> 5) * 64 + r + 16 * ((c & 15) >> 2)) * 8 + ((c & 16) >> 2) + (c & 3);
}
__device__ __forceinline__ int frag16(int c, int t) { return ((c >> 4) * 64 + (c & 15) + 16 * (t >> 2)) * 4 + (t & 3); }
__device__ __forceinline__ int fragkb(int c, int s, int t) { return ((c & 15) + 16 * (t >> 2)) * 8 + 4 * s + (t & 3); }
// Kb^T tiles 0 .. ct/2 - 1 fill the record array at byte lo, the others the one at hi, so the two
// tiles of a 32-channel group are adjacent.
__host__ __device__ constexpr int kb_tile_off(int i, int ct, int lo, int hi) {
    return i < ct / 2 ? lo + 1024 * i : hi + 1024 * (i - ct / 2);
}
__device__ __forceinline__ int fragT(int r, int s) { return (r + 16 * (s >> 2)) * 4 + (s & 3); }

// `base + off` as a pointer whose offset sits in a register the compiler cannot see through,
// while the pointer still derives from `base`: reads through it then address from that register
// with immediate offsets (below 64 KB) instead of forming each address, and alias analysis still
// knows which LDS buffer they read (so no waits for transfers into the other buffer).
template <typename T>
__device__ __forceinline__ T* lds_at(T* base, uint32_t off) {
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    lds_u8* const b = (lds_u8*)(base);
    const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(b));
    uint32_t x = a + off;
    asm volatile("" : "+v"(x));
    return (T*)(b + (x - a));
}

// LDS ordering inside a one-wave workgroup: a wave's LDS operations execute in order, so only the
// compiler must keep them in place.  A wavefront-scope fence does that and emits no wait (a
// workgroup barrier's fence would also wait for every transfer in flight).
__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Token range [bos, end) of sequence n of a packed batch (B = 1, T tokens in all).  The offsets
// are clamped so that 0 <= bos <= end <= T whatever cu_seqlens holds: with malformed offsets
// (negative, past T, decreasing) results are unspecified, but every slot base and buffer range
// derived from bos and end stays inside the buffers sized for T tokens.
__device__ __forceinline__ int64_t seq_start(const ChunkArgs& p, int n) {
    const int64_t a = p.cu[n];
    return a < 0 ? 0 : a > p.T ? p.T : a;
}
__device__ __forceinline__ void seq_bounds(const ChunkArgs& p, int n, int64_t& bos, int64_t& end) {
    bos = seq_start(p, n);
    const int64_t b = p.cu[n + 1];
    end = b < bos ? bos : b > p.T ? p.T : b;
}

// ---- segments of long sequences ---------------------------------------------------------------
// A long sequence is cut into segments of 2^seg_shift tokens [bagrov § Уровень графического
// ускорителя: the long-context scheduler].  The state after a segment is an affine map of the
// state before it, S_out = M S_in + B (M: d_k x d_k, B: d_k x d_v), so every segment's pair can be
// computed at once, the pairs combined along each sequence by a scan, and every later segment run
// again from its true start state.  Segment slots: n * max(1, ceil(T / seg)) for fixed-length
// batches, floor(bos_n / seg) + n for packed ones; per (slot, head) the workspace holds the
// segment's start state, M and B in fp32.
__device__ __forceinline__ int64_t seg_count(int64_t len, int shift) {
    return len <= 0 ? 1 : ((len - 1) >> shift) + 1;   // an empty sequence still has one
}

// Segment slot -> sequence n and segment s within it; false for slots no segment maps to.
__device__ __forceinline__ bool locate_seg(const ChunkArgs& p, const SegArgs& sg, int64_t slot,
                                           int& n, int64_t& s) {
    const int sh = sg.seg_shift;
    if (p.cu) {
        int lo = 0, hi = p.n_seqs - 1;
        while (lo < hi) {                 // largest n with base(n) <= slot
            const int mid = (lo + hi + 1) >> 1;
            const int64_t base = (seq_start(p, mid) >> sh) + mid;
            if (base <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        int64_t bos, end;
        seq_bounds(p, n, bos, end);
        s = slot - ((bos >> sh) + n);
        return s >= 0 && s < seg_count(end - bos, sh);
    }
    const int64_t per = seg_count(p.T, sh);
    n = static_cast<int>(slot / per);
    s = slot % per;
    return n < p.n_seqs;
}

// Launch-local (slot or sequence, head) index k over the launch's heads [head0, head0 + heads)
// -> the global index slot * H + h of the same pair (the identity for a launch over all heads).
__device__ __forceinline__ int64_t global_unit(const ChunkArgs& p, int64_t k) {
    return (k / p.heads) * p.H + p.head0 + k % p.heads;
}

// Length of sequence m's last segment (0 for an empty sequence).
__device__ __forceinline__ int64_t last_seg_len(const ChunkArgs& p, const SegArgs& sg, int m) {
    int64_t bos, end;
    seq_bounds(p, m, bos, end);
    const int64_t len = end - bos;
    return len - ((seg_count(len, sg.seg_shift) - 1) << sg.seg_shift);
}
// Number of segments of a packed batch that are not their sequence's last (all 2^seg_shift tokens).
__device__ __forceinline__ int64_t full_seg_count(const ChunkArgs& p, const SegArgs& sg) {
    int64_t acc = 0;
    for (int m = 0; m < p.n_seqs; ++m) {
        int64_t bos, end;
        seq_bounds(p, m, bos, end);
        acc += seg_count(end - bos, sg.seg_shift) - 1;
    }
    return acc;
}
// The sequences of a packed batch ranked by the length of their last segment, longest first
// (ties in sequence order): order[r] is the sequence of rank r.  Thread t ranks sequence t, so
// the workgroup must have at least n_seqs threads; every thread calls this (it ends in a barrier).
__device__ __forceinline__ void rank_last_segments(const ChunkArgs& p, const SegArgs& sg, int* order) {
    const int t = static_cast<int>(threadIdx.x);
    if (t < p.n_seqs) {
        const int64_t lt = last_seg_len(p, sg, t);
        int r = 0;
        for (int j = 0; j < p.n_seqs; ++j) {
            const int64_t lj = last_seg_len(p, sg, j);
            r += (lj > lt) || (lj == lt && j < t);
        }
        order[r] = t;
    }
    __syncthreads();
}

// Work index k -> sequence n, segment s and its slot, ordered longest first: every sequence's
// segments but its last (all 2^seg_shift tokens), then the last segments (the partial ones) by
// decreasing length when `order` ranks them (rank_last_segments), else in sequence order, so that
// a launch with more workgroups than CUs ends on its shortest ones.  Linear in the number of
// sequences for packed batches (a segmented launch has at most 128 (sequence, head) units).
__device__ __forceinline__ bool locate_seg_lpt(const ChunkArgs& p, const SegArgs& sg, int64_t k,
                                               int& n, int64_t& s, int64_t& slot,
                                               const int* order = nullptr) {
    const int sh = sg.seg_shift;
    if (!p.cu) {
        const int64_t per = seg_count(p.T, sh), full = static_cast<int64_t>(p.n_seqs) * (per - 1);
        if (k < full) {
            n = static_cast<int>(k / (per - 1));
            s = k % (per - 1);
        } else {
            if (k - full >= p.n_seqs) return false;
            n = static_cast<int>(k - full);
            s = per - 1;
        }
        slot = static_cast<int64_t>(n) * per + s;
        return true;
    }
    int64_t acc = 0;
    for (int m = 0; m < p.n_seqs; ++m) {
        int64_t bos, end;
        seq_bounds(p, m, bos, end);
        const int64_t cnt = seg_count(end - bos, sh) - 1;
        if (k < acc + cnt) {
            n = m;
            s = k - acc;
            slot = (bos >> sh) + m + s;
            return true;
        }
        acc += cnt;
    }
    if (k - acc >= p.n_seqs) return false;
    n = order ? order[k - acc] : static_cast<int>(k - acc);
    int64_t bos, end;
    seq_bounds(p, n, bos, end);
    s = seg_count(end - bos, sh) - 1;
    slot = (bos >> sh) + n + s;
    return true;
}

}  // namespace
}  // namespace kda
