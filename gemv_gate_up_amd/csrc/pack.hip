// pack.hip -- builds the fused weight buffers described in geometry.h.
//
// The gate/up packer realises the fused weight W_fused (K x 2N) of
// "Tile-Level Activation Overlap for Efficient LLM Inference" (Kernel-2),
// with gate and up interleaved by blocks of 16 columns instead of single
// columns; the down packer lays Wdown out in the same piece format so that
// the same kernels stream it.  Packing is a pure bit permutation (no
// arithmetic): each output element is one input element or zero padding.
//
// FP8 weights are quantised while packing, column by column (the scheme is
// stated with the DT_FP8W layout): a first pass finds each column's largest
// magnitude and stores scale = amax / 448, a second pass writes the codes of
// w / scale.  Both divisions are IEEE fp32 (__fdiv_rn) and the encoding is
// exact integer arithmetic, so the codes are fully determined by the input.
// MXFP4 weights likewise: block scales first, then the codes of w / 2^s
// (exact: a power-of-two scale).
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

// Column of a packed slot (pair block pb, half h, column c of the half) and
// the source matrix that holds it.
__device__ __forceinline__ int64_t packed_col(int64_t pb, int h, int c, int plain) {
    return plain ? pb * 32 + h * 16 + c : pb * 16 + c;
}

// One thread per packed column slot: scale = max_k |w[k][n]| / 448.
__global__ void __launch_bounds__(256)
fp8_scale_kernel(const uint16_t* __restrict__ src0, const uint16_t* __restrict__ src1,
                 float* __restrict__ scales, int64_t K, int64_t N, int64_t slots, int plain)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= slots)
        return;
    const int64_t pb = t / 32;
    const int h = (int)((t / 16) % 2), c = (int)(t % 16);
    const int64_t n = packed_col(pb, h, c, plain);
    const uint16_t* src = (plain || h == 0) ? src0 : src1;
    float amax = 0.f;
    if (n < N)
        for (int64_t k = 0; k < K; ++k)
            amax = fmaxf(amax, fabsf(bf16_to_f32(src[k * N + n])));
    scales[t] = __fdiv_rn(amax, 448.0f);
}

// E4M3 code of v: nearest value, ties to the even code, saturating at 448.
//   |v| >= 448            -> 0x7E (S.1111.110)
//   |v| <  2^-6           -> subnormal code round(|v| * 2^9), 0..8 (8 is 2^-6)
//   otherwise             -> keep 3 of fp32's 23 mantissa bits, rounding the
//                            other 20 to nearest even (a carry moves into the
//                            exponent), and rebias the exponent from 127 to 7
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return 0x7Fu;                              // NaN stays NaN
    if (a >= 0x43E00000u)                          // 448.0f
        return sign | 0x7Eu;
    if (a < 0x3C800000u)                           // 2^-6
        return sign | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// One thread per 16-byte vector of the FP8 pieces.
__global__ void __launch_bounds__(256)
pack_fp8_kernel(const uint16_t* __restrict__ src0, const uint16_t* __restrict__ src1,
                const float* __restrict__ scales, i32x4* __restrict__ dst, int64_t K, int64_t N,
                int64_t nkc, int64_t total_vecs, int plain)
{
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= total_vecs)
        return;
    const int lane = (int)(v % PIECE_VECS);
    const int64_t piece = v / PIECE_VECS;
    const int h = (int)(piece % 2);
    const int64_t kc = (piece / 2) % nkc;
    const int64_t pb = piece / (2 * nkc);
    const int c = lane % 16, g = lane / 16;
    const int64_t n = packed_col(pb, h, c, plain);
    const uint16_t* src = (plain || h == 0) ? src0 : src1;
    const float s = scales[pb * 32 + h * 16 + c];
    uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int64_t k = kc * 64 + (e < 8 ? g * 8 + e : 32 + g * 8 + (e - 8));
        uint32_t code = 0u;
        if (s != 0.f && k < K && n < N)
            code = e4m3_code(__fdiv_rn(bf16_to_f32(src[k * N + n]), s));
        word[e / 4] |= code << (8 * (e % 4));
    }
    dst[v] = i32x4{(int)word[0], (int)word[1], (int)word[2], (int)word[3]};
}

// MXFP4: one thread per (pair block, k piece, half, column, chunk), in the
// order of the scale table, so thread t writes byte t: the E8M0 code of the
// block's shared exponent floor(log2 amax) - 2, clamped to [-126, 127]
// (code 127, exponent 0, for an all-zero block).  A NaN weight does not
// count toward amax (fmaxf drops it); an infinite amax takes the clamp's
// top, 127.
__global__ void __launch_bounds__(256)
mx_scale_kernel(const uint16_t* __restrict__ src0, const uint16_t* __restrict__ src1,
                uint8_t* __restrict__ scales, int64_t K, int64_t N, int64_t nkc, int64_t total,
                int plain)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total)
        return;
    const int j = (int)(t % 4), c = (int)((t / 4) % 16), h = (int)((t / 64) % 2);
    const int64_t kc = (t / 128) % nkc, pb = t / (128 * nkc);
    const int64_t n = packed_col(pb, h, c, plain);
    const uint16_t* src = (plain || h == 0) ? src0 : src1;
    const int64_t k0 = kc * 128 + j * 32;
    float amax = 0.f;
    if (n < N)
        for (int64_t k = k0; k < k0 + 32 && k < K; ++k)
            amax = fmaxf(amax, fabsf(bf16_to_f32(src[k * N + n])));
    int s = 0;
    if (amax == __builtin_inff()) {
        s = 127;
    } else if (amax > 0.f) {
        int e;
        frexpf(amax, &e);             // amax = f * 2^e, f in [0.5, 1)
        s = e - 1 - 2;
        s = s < -126 ? -126 : (s > 127 ? 127 : s);
    }
    scales[t] = (uint8_t)(s + 127);
}

// E2M1 code of q: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the
// even code (the thresholds below are the midpoints; a tie lands on the
// side whose code is even), saturating at 6; the sign goes to bit 3.  E2M1
// has no infinity or NaN: both fall through every comparison to code 7.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
    const uint32_t sign = (__builtin_bit_cast(uint32_t, q) >> 28) & 8u;
    const float a = fabsf(q);
    uint32_t c;
    if (a <= 0.25f)      c = 0;
    else if (a < 0.75f)  c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f)  c = 3;
    else if (a <= 2.5f)  c = 4;
    else if (a < 3.5f)   c = 5;
    else if (a <= 5.0f)  c = 6;
    else                 c = 7;
    return sign | c;
}

// One thread per 16-byte vector of the MXFP4 pieces.
__global__ void __launch_bounds__(256)
pack_mxfp4_kernel(const uint16_t* __restrict__ src0, const uint16_t* __restrict__ src1,
                  const uint8_t* __restrict__ scales, i32x4* __restrict__ dst, int64_t K,
                  int64_t N, int64_t nkc, int64_t total_vecs, int plain)
{
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= total_vecs)
        return;
    const int lane = (int)(v % PIECE_VECS);
    const int64_t piece = v / PIECE_VECS;       // ((pb * nkc + kc) * 2 + h)
    const int h = (int)(piece % 2);
    const int64_t kc = (piece / 2) % nkc;
    const int64_t pb = piece / (2 * nkc);
    const int c = lane % 16, g = lane / 16;
    const int64_t n = packed_col(pb, h, c, plain);
    const uint16_t* src = (plain || h == 0) ? src0 : src1;
    uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s = (int)scales[piece * 64 + c * 4 + j] - 127;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = kc * 128 + j * 32 + g * 8 + e;
            const float w = (k < K && n < N) ? bf16_to_f32(src[k * N + n]) : 0.f;
            word[j] |= e2m1_code(ldexpf(w, -s)) << (4 * e);
        }
    }
    dst[v] = i32x4{(int)word[0], (int)word[1], (int)word[2], (int)word[3]};
}

// Activations into the packed layout of geometry.h, four 16-byte vectors of
// the output per thread (a workgroup covers 1,024 consecutive vectors, the
// thread's four 256 apart, all four loads issued before the first store): the
// 64 threads of a piece read 16 rows x 64 contiguous bytes and write the
// piece as one 1 KB run.  Vectors of padded rows or K are zero.  K is a
// multiple of 8, so a vector is all valid or all padding.
constexpr int PACK_ACT_VPT = 4;

__global__ void __launch_bounds__(256)
pack_act_kernel(const uint16_t* __restrict__ x, int64_t lda, int64_t M, int64_t K, int64_t nkc,
                uint16_t* __restrict__ dst, int64_t total_vecs)
{
    const int64_t v0 = (int64_t)blockIdx.x * (256 * PACK_ACT_VPT) + threadIdx.x;
    i32x4 val[PACK_ACT_VPT];
    bool ok[PACK_ACT_VPT];
#pragma unroll
    for (int j = 0; j < PACK_ACT_VPT; ++j) {
        const int64_t v = v0 + j * 256;
        const int lane = (int)(v % PIECE_VECS);
        // pieces number at most 2^14 row blocks x 2^15 chunks: 32-bit
        const uint32_t piece = (uint32_t)(v / PIECE_VECS), kcs = (uint32_t)nkc;
        const int64_t row = (int64_t)(piece / kcs) * 16 + lane % 16;
        const int64_t k = (int64_t)(piece % kcs) * 32 + (lane / 16) * 8;
        // every lane loads (padding lanes the first vector of x, then
        // discarded), so the four loads issue back to back without branches
        ok[j] = v < total_vecs && row < M && k < K;
        val[j] = *(const i32x4*)(x + (ok[j] ? row * lda + k : 0));
    }
#pragma unroll
    for (int j = 0; j < PACK_ACT_VPT; ++j) {
        const int64_t v = v0 + j * 256;
        if (v < total_vecs)
            *(i32x4*)(dst + v * 8) = ok[j] ? val[j] : i32x4{0, 0, 0, 0};
    }
}

hipError_t launch_pack_act(const void* x, int64_t lda, int64_t M, int64_t K, int64_t nkc, void* dst,
                           hipStream_t s)
{
    const int64_t total = act_packed_bytes(M, nkc) / 16;
    if (total == 0)
        return hipSuccess;
    pack_act_kernel<<<dim3((unsigned)ceil_div(total, 256 * PACK_ACT_VPT)), dim3(256), 0, s>>>(
        (const uint16_t*)x, lda, M, K, nkc, (uint16_t*)dst, total);
    return hipGetLastError();
}

hipError_t launch_pack(const void* src0, const void* src1, void* dst, const PackGeom& g,
                       int plain, hipStream_t s)
{
    if (g.dt == DT_MXFP4W) {
        uint8_t* scales = (uint8_t*)dst + g.scale_offset();
        const int64_t nsc = g.npb * g.nkc * 2 * 64;
        mx_scale_kernel<<<dim3((unsigned)ceil_div(nsc, 256)), dim3(256), 0, s>>>(
            (const uint16_t*)src0, (const uint16_t*)src1, scales, g.K, g.N, g.nkc, nsc, plain);
        const int64_t total = g.npb * g.nkc * 2 * PIECE_VECS;
        pack_mxfp4_kernel<<<dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s>>>(
            (const uint16_t*)src0, (const uint16_t*)src1, scales, (i32x4*)dst, g.K, g.N, g.nkc,
            total, plain);
        return hipGetLastError();
    }
    if (g.dt == DT_FP8W) {
        float* scales = (float*)((uint8_t*)dst + g.scale_offset());
        const int64_t slots = g.npb * 32;
        fp8_scale_kernel<<<dim3((unsigned)ceil_div(slots, 256)), dim3(256), 0, s>>>(
            (const uint16_t*)src0, (const uint16_t*)src1, scales, g.K, g.N, slots, plain);
        const int64_t total = g.npb * g.nkc * 2 * PIECE_VECS;
        pack_fp8_kernel<<<dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s>>>(
            (const uint16_t*)src0, (const uint16_t*)src1, scales, (i32x4*)dst, g.K, g.N, g.nkc,
            total, plain);
        return hipGetLastError();
    }
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
