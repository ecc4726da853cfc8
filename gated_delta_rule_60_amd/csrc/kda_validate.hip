// kda_validate.hip -- the optional debug check of the inputs' device-resident preconditions,
// enabled by the environment variable KDA_DEBUG_VALIDATE (any value but "" or "0").
//
// The prefill and decode entry points take two things on trust that the host cannot see: the
// log-decay g lies in [-5, 0] -- the bound on the forget gate that keeps every 16-token block's
// decay factors inside the floating range ([habr] "Как устроена Kimi K3: …", § "Последовательность:
// три KDA на один глобальный MLA") -- and a packed batch's cu_seqlens start at 0, never decrease
// and end at the token count.  With the check on, a call first runs small kernels that test them,
// waits for their result (a host synchronisation on the caller's stream) and reports a violation
// as KDA_ERR_INVALID_ARGUMENT before any other work is enqueued.  The result lives in one word
// of library-owned device memory; calls that overlap on one device share it.  Not for use under
// stream capture.
#include <stdlib.h>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

__device__ unsigned int validate_word;   // bit 0: g out of range; bit 1: cu_seqlens malformed

__global__ void clear_word_kernel(unsigned int* w) { *w = 0u; }

template <int DT>
__global__ void __launch_bounds__(256) check_g_kernel(const void* g, int64_t n, unsigned int* w) {
    bool bad = false;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const float x = load_as_f32<DT>(g, i);
        bad |= !(x >= -5.0f && x <= 0.0f);     // NaN fails too
    }
    if (bad) atomicOr(w, 1u);
}

__global__ void check_cu_kernel(const int32_t* cu, int32_t n_seqs, int64_t total, unsigned int* w) {
    bool bad = cu[0] != 0 || static_cast<int64_t>(cu[n_seqs]) != total;
    for (int32_t i = threadIdx.x; i < n_seqs; i += blockDim.x) bad |= cu[i + 1] < cu[i];
    if (bad) atomicOr(w, 2u);
}

}  // namespace

bool debug_validation_enabled() {
    const char* e = getenv("KDA_DEBUG_VALIDATE");
    return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

hipError_t debug_validate(const void* g, int g_dtype, int64_t g_elems, const int32_t* cu,
                          int32_t n_seqs, int64_t total, hipStream_t stream, bool* ok) {
    *ok = true;
    unsigned int* w = nullptr;
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&w), HIP_SYMBOL(validate_word));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, w);
    if (g != nullptr && g_elems > 0) {
        const int64_t blocks = (g_elems + 255) / 256;
        const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
        if (g_dtype == KDA_F32)
            hipLaunchKernelGGL(check_g_kernel<KDA_F32>, dim3(grid), dim3(256), 0, stream, g, g_elems, w);
        else
            hipLaunchKernelGGL(check_g_kernel<KDA_BF16>, dim3(grid), dim3(256), 0, stream, g, g_elems, w);
    }
    if (cu != nullptr)
        hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, total, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    unsigned int host = 0;
    e = hipMemcpyAsync(&host, w, sizeof(host), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return e;
    *ok = (host == 0u);
    return hipSuccess;
}

}  // namespace kda
