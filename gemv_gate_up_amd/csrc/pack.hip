// pack.hip -- builds the fused weight buffers described in geometry.h.
//
// The gate/up packer realises the fused weight W_fused (K x 2N) of
// "Tile-Level Activation Overlap for Efficient LLM Inference" (Kernel-2),
// with gate and up interleaved by blocks of 16 columns instead of single
// columns; the down packer lays Wdown out in the same piece format so that
// the same kernels stream it.  Packing is a pure bit permutation (no
// arithmetic): each output element is one input element or zero padding.
#include "device_common.h"
#include "launch.h"

namespace swg {

// One thread per 16-byte vector of the packed buffer.
//   gate/up: src0 = Wg, src1 = Wu (both K x N row-major), half selects one.
//   down:    src0 = src1 = Wd (K x N row-major), half selects the column block.
template <typename T>
__global__ void __launch_bounds__(256)
pack_kernel(const T* __restrict__ src0, const T* __restrict__ src1, T* __restrict__ dst,
            int64_t K, int64_t N, int64_t nkc, int64_t total_vecs, int plain)
{
    constexpr int VE = 16 / sizeof(T);
    constexpr int KC = 4 * VE;
    int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= total_vecs)
        return;
    int lane = (int)(v % PIECE_VECS);
    int64_t piece = v / PIECE_VECS;
    int half = (int)(piece % 2);
    int64_t kc = (piece / 2) % nkc;
    int64_t pb = piece / (2 * nkc);
    int c = lane % 16, g = lane / 16;
    int64_t n = plain ? pb * 32 + half * 16 + c : pb * 16 + c;
    const T* src = (plain || half == 0) ? src0 : src1;
    T vals[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        int64_t k = kc * KC + g * VE + e;
        vals[e] = (k < K && n < N) ? src[k * N + n] : (T)0;
    }
    T* out = dst + v * VE;
#pragma unroll
    for (int e = 0; e < VE; ++e)
        out[e] = vals[e];
}

hipError_t launch_pack(const void* src0, const void* src1, void* dst, const PackGeom& g,
                       int plain, hipStream_t s)
{
    int64_t total_vecs = g.npb * g.nkc * 2 * PIECE_VECS;
    int64_t blocks = ceil_div(total_vecs, 256);
    if (g.dt == DT_F32)
        pack_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            (const float*)src0, (const float*)src1, (float*)dst, g.K, g.N, g.nkc, total_vecs, plain);
    else
        pack_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            (const uint16_t*)src0, (const uint16_t*)src1, (uint16_t*)dst, g.K, g.N, g.nkc,
            total_vecs, plain);
    return hipGetLastError();
}

}  // namespace swg
