// Test helper (not part of the library): fills the whole 160 KB of LDS that a
// workgroup can hold with one 32-bit pattern, in enough workgroups to visit every
// compute unit, so that a following kernel starts on LDS holding that pattern
// wherever it does not write first. With 0xFFFFFFFF (NaN as fp32 and as both
// bf16 halves), a kernel that reads LDS it never wrote turns its outputs NaN.
#include <hip/hip_runtime.h>

namespace {
constexpr unsigned LDS_BYTES = 160u * 1024u;
constexpr unsigned WORDS = LDS_BYTES / 4u;

__global__ __launch_bounds__(256) void k_lds_fill(unsigned v, unsigned sentinel, unsigned* flag) {
    extern __shared__ unsigned s[];
    for (unsigned i = threadIdx.x; i < WORDS; i += 256u) s[i] = v;
    __syncthreads();
    // never true (sentinel != v); it keeps the stores from being dropped as dead
    if (s[(threadIdx.x * 7u) % WORDS] == sentinel) flag[0] = 1u;
}
}  // namespace

// Queues the fill on `stream`; flag: device buffer of at least one unsigned.
// Returns 0, or 1 if the LDS size attribute or 2 if the launch failed.
extern "C" int lds_fill(unsigned v, unsigned* flag, void* stream) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lds_fill), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)LDS_BYTES) != hipSuccess)
        return 1;
    hipLaunchKernelGGL(k_lds_fill, dim3(2048), dim3(256), LDS_BYTES, static_cast<hipStream_t>(stream), v, v ^ 1u, flag);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
