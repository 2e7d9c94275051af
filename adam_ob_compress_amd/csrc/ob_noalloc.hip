// ob_noalloc.hip -- the static device buffer of the no-allocation compressed step
// (ob_adam_compress_step_noalloc in ob_api.cpp), its per-device address, and the kernel that writes
// the block tables of uniform chunks into it.
//
// Callers that cannot allocate (graph capture, serving loops, harnesses that forbid hipMalloc) still
// need the per-block sums of squares and the block tables a plan would hold.  They live in `scratch`,
// a file-scope device array that every GPU the library runs on holds until the process ends.  Host
// code never passes the array's name to a kernel or a copy: its host-side symbol is only a handle.
// noalloc_scratch() asks the runtime, once per device and with that device current, for the device
// address of that device's copy and keeps it; that address is what the kernels are given.
#include "ob_internal.h"

#include <mutex>

// the buffer: one copy per device, never addressed by this name from host code (see noalloc_scratch)
static __device__ __align__(256) unsigned char scratch[ob::kNoallocScratchBytes];

namespace ob {
namespace {

constexpr int kMaxDevices = 64;

__global__ __launch_bounds__(kBlock) void k_uniform_tables(UniformTables t)
{
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (j < t.n1) t.items1[j] = uniform_item(j, t.n, t.chunk, t.K, t.be1, t.nbf1);
    if (j < t.n2) t.items2[j] = uniform_item(j, t.n, t.chunk, t.K, t.be2, t.nbf2);
    if (j <= t.K) {
        const int32_t c = static_cast<int32_t>(j);
        t.first1[j] = c < t.K ? c * t.nbf1 : static_cast<int32_t>(t.n1);
        t.first2[j] = c < t.K ? c * t.nbf2 : static_cast<int32_t>(t.n2);
        t.off[j] = c < t.K ? static_cast<int64_t>(c) * t.chunk : t.n;
        if (t.ident) t.ident[j] = c;
    }
}

}  // namespace

void* noalloc_scratch(int device)
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[device] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[device] = p;
    }
    return addr[device];
}

hipError_t launch_uniform_tables(const UniformTables& t, hipStream_t s)
{
    int64_t m = t.n1 > t.n2 ? t.n1 : t.n2;
    if (t.K + 1 > m) m = t.K + 1;
    const unsigned grid = static_cast<unsigned>((m + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(k_uniform_tables, dim3(grid), dim3(kBlock), 0, s, t);
    return hipGetLastError();
}

}  // namespace ob
