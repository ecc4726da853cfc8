// kda_gate.hip -- forget-gate log-decay g = g_min * sigmoid(exp(A) * z), one pass over z.
//
// Page: "Как устроена Kimi K3: 2,8 трлн параметров, линейное внимание и агенты на миллион
// токенов" (savepearlharbor.com), § "Последовательность: три KDA на один глобальный MLA":
// the forget factor is alpha = exp(g) with g = g_min * sigmoid(exp(A) * z) and g_min = -5.
//
// Pure streaming work (6 bytes per element for bf16 z -> fp32 g): each lane handles four
// consecutive channels per step with 8/16-byte loads and stores, grid-stride over the tensor.  The
// grid is sized so that the stride keeps a lane on the same channels where it can, and a lane
// forms a channel's rate (an fp64 exp) only when its channels change.
#include "kda_common.hpp"
#include "kda_internal.hpp"

#include <numeric>

namespace kda {

template <int ZDT, int GDT>
__global__ void __launch_bounds__(256) gate_kernel_vec4(const float* __restrict__ A,
                                                        const void* __restrict__ z,
                                                        void* __restrict__ g, int64_t n_vec,
                                                        int32_t H, int32_t dk, float g_min) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int32_t hdk = H * dk;
    int32_t cached = -1;
    GateRate r[4];
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_vec;
         i += stride) {
        const int64_t e = i * 4;                      // first element of this group of four
        const int32_t ac = static_cast<int32_t>(e % hdk);  // (head, channel) index into A
        if (ac != cached) {
            const float4 aa = *reinterpret_cast<const float4*>(A + ac);
            r[0] = gate_rate(aa.x); r[1] = gate_rate(aa.y); r[2] = gate_rate(aa.z); r[3] = gate_rate(aa.w);
            cached = ac;
        }
        const float4 zz = load4_as_f32<ZDT>(z, e);
        float4 out;
        out.x = gate_log_decay(r[0], zz.x, g_min);
        out.y = gate_log_decay(r[1], zz.y, g_min);
        out.z = gate_log_decay(r[2], zz.z, g_min);
        out.w = gate_log_decay(r[3], zz.w, g_min);
        store4_from_f32<GDT>(g, e, out);
    }
}

template <int ZDT, int GDT>
__global__ void __launch_bounds__(256) gate_kernel_scalar(const float* __restrict__ A,
                                                          const void* __restrict__ z,
                                                          void* __restrict__ g, int64_t n,
                                                          int32_t H, int32_t dk, float g_min) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int32_t hdk = H * dk;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += stride) {
        const float a = A[e % hdk];
        store_from_f32<GDT>(g, e, gate_log_decay(gate_rate(a), load_as_f32<ZDT>(z, e), g_min));
    }
}

template <int ZDT, int GDT>
static hipError_t launch_gate_t(const float* A, const void* z, void* g, int64_t n_tokens,
                                int32_t H, int32_t dk, float g_min, hipStream_t stream) {
    const int64_t n = n_tokens * H * dk;
    const int threads = 256;
    // Enough blocks to fill 256 CUs several times over; the loop strides over the rest.
    const int64_t max_blocks = 256 * 16;
    const bool vec = (dk % 4 == 0) && (reinterpret_cast<uintptr_t>(A) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(z) % (ZDT == KDA_F32 ? 16 : 8) == 0) &&
                     (reinterpret_cast<uintptr_t>(g) % (GDT == KDA_F32 ? 16 : 8) == 0);
    if (vec) {
        const int64_t n_vec = n / 4;
        int64_t blocks = std::min<int64_t>((n_vec + threads - 1) / threads, max_blocks);
        // a stride that is a multiple of the groups per token keeps each lane on its channels
        const int64_t groups = H * dk / 4;
        const int64_t q = groups / std::gcd<int64_t>(groups, threads);
        if (blocks * threads < n_vec && q <= max_blocks) blocks = blocks / q * q;
        hipLaunchKernelGGL((gate_kernel_vec4<ZDT, GDT>), dim3(static_cast<unsigned>(blocks)),
                           dim3(threads), 0, stream, A, z, g, n_vec, H, dk, g_min);
    } else {
        const int64_t blocks = std::min<int64_t>((n + threads - 1) / threads, max_blocks);
        hipLaunchKernelGGL((gate_kernel_scalar<ZDT, GDT>), dim3(static_cast<unsigned>(blocks)),
                           dim3(threads), 0, stream, A, z, g, n, H, dk, g_min);
    }
    return hipGetLastError();
}

hipError_t launch_gate(const float* A, const void* z, int z_dtype, void* g, int g_dtype,
                       int64_t n_tokens, int32_t H, int32_t dk, float g_min, hipStream_t stream) {
    if (z_dtype == KDA_BF16 && g_dtype == KDA_F32)
        return launch_gate_t<KDA_BF16, KDA_F32>(A, z, g, n_tokens, H, dk, g_min, stream);
    if (z_dtype == KDA_BF16 && g_dtype == KDA_BF16)
        return launch_gate_t<KDA_BF16, KDA_BF16>(A, z, g, n_tokens, H, dk, g_min, stream);
    if (z_dtype == KDA_F32 && g_dtype == KDA_F32)
        return launch_gate_t<KDA_F32, KDA_F32>(A, z, g, n_tokens, H, dk, g_min, stream);
    return launch_gate_t<KDA_F32, KDA_BF16>(A, z, g, n_tokens, H, dk, g_min, stream);
}

}  // namespace kda
