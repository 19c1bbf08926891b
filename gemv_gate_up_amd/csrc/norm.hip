// norm.hip -- RMSNorm prologue of the MLP block: n = r / sqrt(mean(r^2) +
// eps) * gamma per row ("Anatomie d'un transformeur sur GPU", §1.1 layer
// skeleton: the normalisation before Wgate/Wup; §1.6 kernel 7).  The pages
// name the operation without its formula; this is the usual RMS form with a
// learned gain and a caller-given eps.
//
// One workgroup per row.  Each thread sums the squares of a strided subset
// of the row in fp32; the 256 partial sums are added by a fixed shuffle tree
// in each wave and then in wave order, so the result does not depend on
// timing.  1 / sqrt uses correctly rounded fp32 square root and division.
// The normalised row is rounded once to the activation type (bf16 or fp32)
// and feeds the gate/up product: row-major, or (bf16, for the many-rows
// path) directly in the packed activation layout of geometry.h, in which
// case the grid also covers the padding rows and each workgroup writes the
// zero K padding of its row.
#include "device_common.h"
#include "launch.h"

namespace swg {

constexpr int NORM_THREADS = 256;

template <typename T>
__global__ void __launch_bounds__(NORM_THREADS)
rmsnorm_kernel(const T* __restrict__ r, const T* __restrict__ gamma, float eps, int64_t M,
               int64_t d, T* __restrict__ n, int64_t packed_nkc)
{
    constexpr int VE = 16 / sizeof(T);
    const int64_t row = blockIdx.x;
    const int64_t nvec = d / VE;
    // destination of vector v (elements v*VE ..) of this row
    auto dst = [&](int64_t v) {
        return packed_nkc > 0 ? n + act_packed_index(row, v * VE, packed_nkc) : n + row * d + v * VE;
    };
    if (row >= M) {   // padding row of the packed layout
        for (int64_t v = threadIdx.x; v < packed_nkc * 32 / VE; v += NORM_THREADS)
            *(i32x4*)dst(v) = i32x4{0, 0, 0, 0};
        return;
    }
    const T* rr = r + row * d;
    float ss = 0.f;
    for (int64_t v = threadIdx.x; v < nvec; v += NORM_THREADS) {
        const i32x4 raw = *(const i32x4*)(rr + v * VE);
        const T* e = (const T*)&raw;
#pragma unroll
        for (int k = 0; k < VE; ++k) {
            const float x = load_act(e + k);
            ss = __builtin_fmaf(x, x, ss);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        ss += __shfl_xor(ss, off);
    __shared__ float part[NORM_THREADS / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NORM_THREADS / 64; ++w)
        tot += part[w];
    const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(tot, (float)d) + eps));
    for (int64_t v = threadIdx.x; v < nvec; v += NORM_THREADS) {
        const i32x4 raw = *(const i32x4*)(rr + v * VE);
        const i32x4 graw = *(const i32x4*)(gamma + v * VE);
        const T* e = (const T*)&raw;
        const T* g = (const T*)&graw;
        i32x4 o;
        T* oe = (T*)&o;
#pragma unroll
        for (int k = 0; k < VE; ++k)
            store_out(oe + k, load_act(e + k) * inv * load_act(g + k));
        *(i32x4*)dst(v) = o;
    }
    for (int64_t v = nvec + threadIdx.x; v < packed_nkc * 32 / VE; v += NORM_THREADS)
        *(i32x4*)dst(v) = i32x4{0, 0, 0, 0};
}

hipError_t launch_rmsnorm(const void* r, const void* gamma, float eps, int64_t M, int64_t d,
                          int dt, void* n, int64_t packed_nkc, hipStream_t s)
{
    if (dt == DT_F32) {
        if (packed_nkc > 0)
            return hipErrorInvalidValue;
        rmsnorm_kernel<float><<<dim3((unsigned)M), dim3(NORM_THREADS), 0, s>>>(
            (const float*)r, (const float*)gamma, eps, M, d, (float*)n, 0);
    } else {
        const int64_t rows = packed_nkc > 0 ? round_up(M, 16) : M;
        rmsnorm_kernel<uint16_t><<<dim3((unsigned)rows), dim3(NORM_THREADS), 0, s>>>(
            (const uint16_t*)r, (const uint16_t*)gamma, eps, M, d, (uint16_t*)n, packed_nkc);
    }
    return hipGetLastError();
}

}  // namespace swg
