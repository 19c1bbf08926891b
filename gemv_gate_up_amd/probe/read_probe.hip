// read_probe.hip -- measurement aids for bench.py, not part of the library's
// C ABI (built as its own libswiglu_probe.so):
//   * a plain streaming read of device memory: the HBM rate a kernel can
//     reach on this board at a given size, reported beside the published
//     peak as the achievable-bandwidth reference of a memory-bound kernel;
//   * the device's compute-unit count and maximum graphics clock, from which
//     bench.py derives the dense bf16 matrix peak at run time.
//
//   int probe_read(const void* p, int64_t nbytes, int* sink, int grid, int u,
//                  hipStream_t stream)
//       grid-stride read of nbytes (a multiple of 16) at device pointer p by
//       `grid` workgroups of 256 threads, each keeping u (4, 8 or 16)
//       nontemporal 16-byte loads in flight; every thread writes one int of
//       `sink` (grid * 256 ints) so that no load is dropped.  Returns a HIP
//       error code (0 on success).
//   int probe_device(int* cus, int* max_clock_khz)
//       of the current device; returns a HIP error code.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) int i32x4;

template <int U>
__global__ void __launch_bounds__(256)
read_kernel(const i32x4* __restrict__ p, int64_t nvec, int* __restrict__ sink)
{
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int acc = 0;
    int64_t v = tid;
    for (; v + (U - 1) * stride < nvec; v += U * stride) {
        i32x4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            r[u] = __builtin_nontemporal_load(p + v + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
    }
    for (; v < nvec; v += stride) {
        const i32x4 r = __builtin_nontemporal_load(p + v);
        acc ^= r.x ^ r.y ^ r.z ^ r.w;
    }
    sink[tid] = acc;
}

extern "C" int probe_read(const void* p, int64_t nbytes, int* sink, int grid, int u,
                          hipStream_t s)
{
    if (!p || !sink || nbytes <= 0 || nbytes % 16 != 0 || grid <= 0)
        return (int)hipErrorInvalidValue;
    const int64_t nvec = nbytes / 16;
    if (u == 4)
        read_kernel<4><<<grid, 256, 0, s>>>((const i32x4*)p, nvec, sink);
    else if (u == 8)
        read_kernel<8><<<grid, 256, 0, s>>>((const i32x4*)p, nvec, sink);
    else if (u == 16)
        read_kernel<16><<<grid, 256, 0, s>>>((const i32x4*)p, nvec, sink);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

extern "C" int probe_device(int* cus, int* max_clock_khz)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, dev);
    return (int)e;
}
