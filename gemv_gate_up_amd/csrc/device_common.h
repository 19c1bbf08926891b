// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.h"

namespace swg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((address_space(3))) void lds_void_t;

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// SiLU (Swish, beta = 1): z * sigmoid(z) = z / (1 + e^-z), with the
// hardware reciprocal (about 1 ulp; an IEEE division costs about four times
// the instructions, and the result is rounded to bf16 or checked at 1e-4
// relative in fp32).  Tends to z for large z and to -0 for very negative z
// (1 + e^-z overflows to inf, whose reciprocal is 0) without producing NaN.
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

template <typename T>
__device__ __forceinline__ float load_act(const T* p);
template <>
__device__ __forceinline__ float load_act<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// Epilogue additions of a plain product (the down projection of the MLP
// block): the bias of the "Affine" operation, then the residual, both in
// fp32 before the one rounding of the store.  Null pointers add nothing.
template <typename T>
__device__ __forceinline__ float plain_tail(float v, const T* resid, int64_t ldr, const T* bias,
                                            int64_t row, int64_t col) {
    if (bias)
        v += load_act(bias + col);
    if (resid)
        v += load_act(resid + row * ldr + col);
    return v;
}

// Buffer resource over [base, base + num_bytes): loads at offsets at or
// past num_bytes return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}

__device__ __forceinline__ i32x4 load_nt16(const i32x4* p) {
    return __builtin_nontemporal_load(p);
}

}  // namespace swg
