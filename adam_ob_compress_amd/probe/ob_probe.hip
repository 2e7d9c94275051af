// ob_probe.hip -- measurement support for bench.py, not part of the optimizer library: a plain copy
// kernel whose HBM traffic is known exactly (n_bytes read, n_bytes written), with the same 16-byte
// lanes and nontemporal loads and stores as the library's streaming kernels.  Its FETCH_SIZE and
// WRITE_SIZE counter readings calibrate the counters for those access kinds; the torch copy the
// bench also runs calibrates them for ordinary accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kPerThread = 4;   // 16-byte vectors per thread per block

template <bool NT>
__global__ __launch_bounds__(kBlock) void k_probe_copy(const f4* __restrict__ src, f4* __restrict__ dst, int64_t nv)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kBlock * kPerThread + threadIdx.x;
    f4 v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t i = base + static_cast<int64_t>(k) * kBlock;
        if (i < nv) v[k] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t i = base + static_cast<int64_t>(k) * kBlock;
        if (i < nv) {
            if (NT)
                __builtin_nontemporal_store(v[k], dst + i);
            else
                dst[i] = v[k];
        }
    }
}

}  // namespace

// Copy n_bytes (a multiple of 16; both pointers 16-byte aligned, device memory) from src to dst on
// `stream`; nontemporal != 0 uses nontemporal loads and stores.  Returns 0, 1 for bad arguments, or
// 2 for a failed launch.
extern "C" int ob_probe_copy(const void* src, void* dst, int64_t n_bytes, int nontemporal, hipStream_t stream)
{
    if (!src || !dst || n_bytes < 0 || n_bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
        reinterpret_cast<uintptr_t>(dst) % 16)
        return 1;
    const int64_t nv = n_bytes / 16;
    if (nv == 0) return 0;
    const int64_t blocks = (nv + kBlock * kPerThread - 1) / (kBlock * kPerThread);
    (void)hipGetLastError();
    if (nontemporal)
        hipLaunchKernelGGL(k_probe_copy<true>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream,
                           static_cast<const f4*>(src), static_cast<f4*>(dst), nv);
    else
        hipLaunchKernelGGL(k_probe_copy<false>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream,
                           static_cast<const f4*>(src), static_cast<f4*>(dst), nv);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
