// geometry.h -- packed weight layout shared by the packer and the kernels.
//
// The gate and up weights are fused into one buffer so that a single stream
// of 16-byte loads feeds both products (the interleaved fused weight of
// "Tile-Level Activation Overlap for Efficient LLM Inference", Kernel-2,
// with column blocks instead of single columns).
//
// Unit of the layout: a "piece" of 1 KB = 64 lanes x 16 bytes.  Lane l of a
// piece holds, for column c = l % 16 of a 16-column block and k-group
// g = l / 16, the VE consecutive K values k0 + g*VE .. k0 + g*VE + VE - 1
// (VE = 8 for bf16, 4 for fp32).  A piece therefore covers 16 columns by
// KC = 4*VE values of K, and it is exactly the B operand of one
// v_mfma_f32_16x16x32_bf16 for bf16 (verified lane layout), loaded with one
// coalesced 16-byte access per lane.
//
// Pieces are grouped in "pair blocks" of two 16-column halves:
//   gate/up buffer: pair block p, half 0 = gate columns 16p..16p+15,
//                                  half 1 = up   columns 16p..16p+15
//   down buffer:    pair block p, half h = output columns 32p+16h..32p+16h+15
// and ordered [pair block][k chunk][half][lane], so one pair block over a
// K range is one contiguous run of 2 KB per chunk.
//
// Padding: K is rounded up to a multiple of KALIGN (two chunks) and the
// number of pair blocks up to a multiple of PB_ALIGN; padded weights are
// zero, so padded products are exactly zero.
//
// FP8 weights (DT_FP8W: OCP E4M3 codes, bf16 activations and outputs): a
// lane's 16 bytes are 16 codes of one column, the 8 K values of its k-group
// in each of two consecutive 32-K chunks (bytes 0-7: k0 + g*8 + 0..7,
// bytes 8-15: k0 + 32 + g*8 + 0..7), so one piece covers 16 columns by 64 K
// and widens into the B operands of two bf16 MFMAs.  K is padded to 64.
// After the pieces comes one fp32 scale per packed column, ordered
// [pair block][half][16] (entry 32p + 16h + c), zero for padded columns.
//
// MXFP4 weights (DT_MXFP4W: OCP MX E2M1 codes with one E8M0 scale per 32
// consecutive K values of a column): a lane's 16 bytes hold, for each of
// four consecutive 32-K chunks j, the 8 values of its k-group (byte 4j + i
// holds k0 + 32j + 8g + 2i in its low nibble and the next K value in its
// high nibble), so one piece covers 16 columns by 128 K and widens into the
// B operands of four MFMAs; each chunk of a column is exactly one MX block.
// K is padded to 128.  After the pieces come the block scales, 64 bytes per
// piece ordered [pair block][k piece][half][column c][chunk j], so that lane
// l reads the four scales of its column as one dword.
#pragma once
#include <stdint.h>

namespace swg {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8W = 2, DT_MXFP4W = 3 };
enum : int { EPI_SWIGLU = 0, EPI_PLAIN = 1 };

constexpr int PIECE_BYTES = 1024;
constexpr int PIECE_VECS = 64;     // 16-byte vectors per piece
constexpr int PB_ALIGN = 8;        // pair blocks: multiple of 8 (256 packed columns)

// Activation (x, h, out, y) element size and 16-byte vector width: bf16 for
// both the bf16 and the FP8-weight types.
__host__ __device__ constexpr inline int elem_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }
__host__ __device__ constexpr inline int act_vec_elems(int dt) { return dt == DT_F32 ? 4 : 8; }
// K covered by one piece, and the K padding.
__host__ __device__ constexpr inline int chunk_k(int dt) {
    return dt == DT_F32 ? 16 : (dt == DT_BF16 ? 32 : (dt == DT_FP8W ? 64 : 128));
}
__host__ __device__ constexpr inline int k_align(int dt) {
    return dt == DT_FP8W || dt == DT_MXFP4W ? chunk_k(dt) : 2 * chunk_k(dt);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Geometry of one packed operand: K is the contraction length, cols_per_pb
// is 16 for gate/up (one output column block per pair) and 32 for down.
struct PackGeom {
    int64_t K;          // valid contraction length
    int64_t N;          // valid output columns
    int64_t nkc;        // chunks of KC along K (padded, even)
    int64_t npb;        // pair blocks (padded to PB_ALIGN)
    int64_t npb_valid;  // pair blocks that hold real columns
    int cols_per_pb;    // output columns per pair block (16 or 32)
    int dt;
    __host__ __device__ int64_t piece_bytes() const { return npb * nkc * 2 * PIECE_BYTES; }
    // FP8 and MXFP4 weights: the scales follow the pieces
    __host__ __device__ int64_t scale_offset() const { return piece_bytes(); }
    __host__ __device__ int64_t bytes() const {
        return piece_bytes() + (dt == DT_FP8W ? npb * 32 * 4 : 0) +
               (dt == DT_MXFP4W ? npb * nkc * 2 * 64 : 0);
    }
    // output row width when the result is kept padded (workspace h)
    __host__ __device__ int64_t padded_cols() const { return npb * cols_per_pb; }
};

// Fused gate/up weight: contraction over d, dff output columns.
__host__ __device__ inline PackGeom gateup_geom(int64_t d, int64_t dff, int dt) {
    PackGeom g;
    g.K = d;
    g.N = dff;
    g.nkc = round_up(d, k_align(dt)) / chunk_k(dt);
    g.npb_valid = ceil_div(dff, 16);
    g.npb = round_up(g.npb_valid, PB_ALIGN);
    g.cols_per_pb = 16;
    g.dt = dt;
    return g;
}

// Packed activations (bf16, many-rows path).  The left operand of the MFMA
// GEMM, M x K, laid out as its A fragments: pieces ordered [row block of 16]
// [32-K chunk], and lane l of a piece holding row l % 16 and the 8
// consecutive K values of k-group l / 16 of its chunk, i.e. element (row, k)
// at index ((row / 16) * nkc + k / 32) * 512 + ((k % 32) / 8 * 16 + row % 16)
// * 8 + k % 8.  Rows are padded to a multiple of 16 and K to the nkc chunks
// of the weight that consumes it; padding is zero.  A piece is one
// contiguous 1 KB load, where a row-major tile row is a 64-byte fragment of
// a line per K step.
__host__ __device__ inline int64_t act_packed_bytes(int64_t M, int64_t nkc) {
    return ceil_div(M, 16) * nkc * PIECE_BYTES;
}
__host__ __device__ inline int64_t act_packed_index(int64_t row, int64_t k, int64_t nkc) {
    return ((row / 16) * nkc + k / 32) * 512 + ((k % 32) / 8 * 16 + row % 16) * 8 + k % 8;
}

// Down weight: contraction over dff, d output columns.
__host__ __device__ inline PackGeom down_geom(int64_t d, int64_t dff, int dt) {
    PackGeom g;
    g.K = dff;
    g.N = d;
    g.nkc = round_up(dff, k_align(dt)) / chunk_k(dt);
    g.npb_valid = ceil_div(d, 32);
    g.npb = round_up(g.npb_valid, PB_ALIGN);
    g.cols_per_pb = 32;
    g.dt = dt;
    return g;
}

}  // namespace swg
