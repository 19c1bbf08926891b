// launch.h -- internal host-side launchers (C++ linkage, not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.h"

namespace swg {

// Packing (pack.hip).  plain = 0: gate/up (src0 = Wg, src1 = Wu);
// plain = 1: down (src0 = src1 = Wd).
hipError_t launch_pack(const void* src0, const void* src1, void* dst, const PackGeom& g,
                       int plain, hipStream_t s);

// Work description for one product of the hot path: out = epi(A . Wpacked).
struct GemmArgs {
    const void* a;      // activations, M x lda row-major (x, or h in the workspace)
    int64_t lda;        // row stride of a in elements
    int a_packed;       // wide path: a is in the packed activation layout (lda unused)
    const void* w;      // packed weights
    PackGeom geom;      // geometry of w
    void* out;          // output, M x ldo row-major
    int64_t ldo;        // row stride of out in elements
    int64_t out_nkc;    // > 0, wide path: out is written in the packed activation layout
                        // with this many 32-K chunks (ldo unused); see geometry.h
    int64_t ncols_out;  // output columns to store (valid columns, or the padded width)
    int64_t M;
    int epi;            // EPI_SWIGLU or EPI_PLAIN
    int dt;
    // EPI_PLAIN only, may be null: out = A.W (+ bias[col]) (+ resid[row][col])
    const void* resid;  // M x ldr, activation type
    int64_t ldr;
    const void* bias;   // ncols_out values, activation type
};

// Packs M x K bf16 activations (row stride lda) into the packed activation
// layout with nkc chunks (pack.hip).
hipError_t launch_pack_act(const void* x, int64_t lda, int64_t M, int64_t K, int64_t nkc, void* dst,
                           hipStream_t s);

// RMSNorm prologue (norm.hip): n = r / sqrt(mean(r^2) + eps) * gamma per
// row; r, gamma and n in the activation type of dt.  packed_nkc > 0 (bf16
// only): n is written in the packed activation layout with that many chunks.
hipError_t launch_rmsnorm(const void* r, const void* gamma, float eps, int64_t M, int64_t d,
                          int dt, void* n, int64_t packed_nkc, hipStream_t s);

// Split-K plan for the skinny kernels.
struct SkinnyPlan {
    int splits;             // K splits across workgroups (1 = epilogue in the same kernel)
    int64_t chunks_per_split;
    int64_t grid_pb;        // pair blocks covered by the grid
    int pb_per_wg;          // pair blocks per workgroup (bf16: 1 or 2)
    int row_tile;           // rows per workgroup row group (bf16: 16*MT, fp32: 8)
    int64_t row_groups;
};

SkinnyPlan plan_skinny(const GemmArgs& g, int num_cus);
size_t skinny_partial_bytes(const GemmArgs& g, const SkinnyPlan& p);

// Skinny path (skinny.hip): weights split over workgroups, fp32 accumulation.
hipError_t launch_skinny(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s);
// Second pass of a split product (skinny.hip): out = epi(sum of `splits`
// fp32 slices of partial, [slice][row][packed column], in slice order).
hipError_t launch_splitk_reduce(const GemmArgs& g, int splits, const float* partial, hipStream_t s);

// Fused down projection (fused.hip): y = (silu(x.Wg) * (x.Wu)) . Wd with
// each workgroup owning a slice of d_ff: it forms its slice of h in LDS and
// writes the slice's fp32 contribution to y; the second pass adds the
// slices in order and applies dn's epilogue (bias, residual).  bf16 only.
struct FusedPlan {
    int mt;          // 16-row tiles per row group (1..4)
    int g;           // gate/up pair blocks per d_ff slice
    int64_t slices;  // d_ff slices = partial slices of y
    int64_t row_groups;
};
FusedPlan plan_fused(const GemmArgs& up, const GemmArgs& dn);
size_t fused_partial_bytes(const GemmArgs& dn, const FusedPlan& p);
hipError_t launch_fused(const GemmArgs& up, const GemmArgs& dn, const FusedPlan& p, float* partial,
                        hipStream_t s);

// Wide path (wide.hip): bf16 MFMA GEMM with LDS double buffering.
hipError_t launch_wide(const GemmArgs& g, hipStream_t s);
// Two-pass (gate K loop, then up K loop) schedule; gate/up products only.
hipError_t launch_wide_phased(const GemmArgs& g, hipStream_t s);
int wide_supported(const GemmArgs& g);
// Workgroups the wide launch of this product would use (for the dispatcher).
int64_t wide_grid_tiles(const GemmArgs& g);
// Sets the launch attributes of every wide instantiation (host calls only);
// done before a stream capture so that none of them is recorded inside it.
hipError_t wide_prepare();

}  // namespace swg
