// fused.hip -- the MLP with the down projection fused into the gate/up
// kernel, for few rows:
//
//     y = sum over d_ff slices s of  h_s . Wd[s rows, :],
//     h_s = silu(x . Wg[:, s]) * (x . Wu[:, s])
//
// The fusion that "Où part le temps d'un token" proposes in its section on
// what remains (the launches): fewer kernels, each longer; and the layer's
// gate/up -> SwiGLU -> down kernels of "Anatomie d'un transformeur sur GPU"
// (§1.6) in one pass.  Each workgroup owns one slice of d_ff (G pair blocks
// of the packed gate/up weight, 16 G columns of h) and one group of up to 64
// rows:
//   1. its waves split the K range of x . [Wg | Wu] over the slice's pair
//      blocks (16-byte nontemporal weight loads, the activations as the
//      16-row A operand of v_mfma_f32_16x16x32_bf16), the wave sums are
//      added in LDS in wave order, and h = silu(g) * u is rounded once to
//      bf16 and kept in LDS laid out as the A operand of the next product:
//      the slice of h never reaches memory;
//   2. its waves split the output columns of y: each multiplies the slice
//      of h by the matching 16 G rows of the packed Wdown and stores that
//      fp32 contribution to y in the workspace;
//   3. the second pass of the split products adds the slices in ascending
//      order and applies the epilogue (bias, residual of the MLP block): the
//      fixed-order, atomic-free reduction of "Un kernel pour les matrices
//      étroites", so results are reproducible run to run.
// What this trades: the h round trip (2 M d_ff bytes written and read back)
// and the separate down-product kernels, against M d 4 bytes of partial y
// per slice, written and read once.
#include "device_common.h"
#include "launch.h"

namespace swg {

constexpr int FU_WAVES = 8;

// MT 16-row tiles per row group, G gate/up pair blocks per d_ff slice, U
// K chunks in flight per wave in the gate/up loop, UD down pair blocks in
// flight per wave in the down loop.
template <int MT, int G, int U, int UD>
__global__ void __launch_bounds__(FU_WAVES * 64)
mlp_fused_kernel(const uint16_t* __restrict__ x, int64_t lda, int64_t d,
                 const i32x4* __restrict__ wp, int64_t nkc_up, int64_t npb_up,
                 const i32x4* __restrict__ wdp, int64_t nkc_dn, int64_t npb_dn_valid,
                 float* __restrict__ partial, int64_t npc, int M)
{
    static_assert(G % 2 == 0 && G * MT <= 16, "a slice is whole 32-K chunks of h; accumulators");
    constexpr int NWV = FU_WAVES;
    constexpr int HC = G / 2;   // 32-K chunks of the down product in one slice
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t slice = blockIdx.x;
    const int64_t pb0 = slice * G;
    const int rbase = blockIdx.z * 16 * MT;
    const int arow = lane & 15;
    const int akoff = (lane >> 4) * 8;

    // ---- 1. gate/up over the slice, waves interleaved over K chunks
    f32x4 accg[G][MT], accu[G][MT];
#pragma unroll
    for (int p = 0; p < G; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            accg[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    const i32x4* wpl = wp + pb0 * nkc_up * 2 * PIECE_VECS + lane;
    for (int64_t kb = wave; kb < nkc_up; kb += NWV * U) {
        i32x4 wg[G][U], wu[G][U], xa[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kc = kb + NWV * u;
#pragma unroll
            for (int p = 0; p < G; ++p) {
                // pair blocks past the packed buffer (a last slice that
                // overhangs it) hold no weights: zero
                if (kc < nkc_up && pb0 + p < npb_up) {
                    wg[p][u] = load_nt16(wpl + (p * nkc_up * 2 + kc * 2) * PIECE_VECS);
                    wu[p][u] = load_nt16(wpl + (p * nkc_up * 2 + kc * 2 + 1) * PIECE_VECS);
                } else {
                    wg[p][u] = i32x4{0, 0, 0, 0};
                    wu[p][u] = i32x4{0, 0, 0, 0};
                }
            }
            const int64_t k = kc * 32 + akoff;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = rbase + mt * 16 + arow;
                xa[u][mt] = (kc < nkc_up && row < M && k < d)
                                ? *(const i32x4*)(x + (int64_t)row * lda + k)
                                : i32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int p = 0; p < G; ++p)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, xa[u][mt]);
                    accg[p][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        av, __builtin_bit_cast(bf16x8, wg[p][u]), accg[p][mt], 0, 0, 0);
                    accu[p][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        av, __builtin_bit_cast(bf16x8, wu[p][u]), accu[p][mt], 0, 0, 0);
                }
    }

    // Wave sums added in LDS in wave order, one pair block at a time; the
    // first 256 threads each finish one (row r, column c) of the 16 x 16
    // tiles of every row tile.  MFMA result layout: lane l holds rows
    // 4 (l / 16) + i of column l % 16.  h goes to hs as the A operand of the
    // down product: [row tile][32-K chunk][lane][8], lane l holding row
    // l % 16 and the 8 h columns of k-group l / 16 of the chunk.
    __shared__ float red[NWV][MT][2][64 * 4];
    __shared__ __attribute__((aligned(16))) uint16_t hs[MT][HC][64 * 8];
    const int t = threadIdx.x;
    const int r = t >> 4, c = t & 15;
    const int src = ((r >> 2) * 16 + c) * 4 + (r & 3);
#pragma unroll
    for (int p = 0; p < G; ++p) {
        if (p > 0)
            __syncthreads();   // the previous pair block's sums have been read
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[wave][mt][0][lane * 4 + i] = accg[p][mt][i];
                red[wave][mt][1][lane * 4 + i] = accu[p][mt][i];
            }
        __syncthreads();
        if (t < 256) {
            // h column 16 p + c of the slice: chunk p / 2, k-group
            // ((p % 2) * 16 + c) / 8, element c % 8
            const int kk = (p % 2) * 16 + c;
            const int hl = (kk >> 3) * 16 + r;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int wv = 0; wv < NWV; ++wv) {
                    g += red[wv][mt][0][src];
                    u += red[wv][mt][1][src];
                }
                hs[mt][p / 2][hl * 8 + (kk & 7)] = f32_to_bf16(silu(g) * u);
            }
        }
    }
    __syncthreads();

    // ---- 2. the slice's contribution to y: waves interleaved over the down
    // product's pair blocks (32 output columns each), UD at a time
    const int64_t kc0 = slice * HC;   // first chunk of the slice in the packed Wdown
    float* pslice = partial + slice * (int64_t)M * npc;
    for (int64_t db = wave; db < npb_dn_valid; db += NWV * UD) {
        i32x4 wd[UD][HC][2];
#pragma unroll
        for (int ud = 0; ud < UD; ++ud) {
            const int64_t dpb = db + NWV * ud;
#pragma unroll
            for (int ch = 0; ch < HC; ++ch)
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    wd[ud][ch][half] = (dpb < npb_dn_valid && kc0 + ch < nkc_dn)
                                           ? load_nt16(wdp + ((dpb * nkc_dn + kc0 + ch) * 2 + half) *
                                                                 PIECE_VECS + lane)
                                           : i32x4{0, 0, 0, 0};
        }
        f32x4 acc[UD][2][MT];
#pragma unroll
        for (int ud = 0; ud < UD; ++ud)
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[ud][half][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ch = 0; ch < HC; ++ch)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8 hv = *(const bf16x8*)&hs[mt][ch][lane * 8];
#pragma unroll
                for (int ud = 0; ud < UD; ++ud)
#pragma unroll
                    for (int half = 0; half < 2; ++half)
                        acc[ud][half][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            hv, __builtin_bit_cast(bf16x8, wd[ud][ch][half]), acc[ud][half][mt],
                            0, 0, 0);
            }
#pragma unroll
        for (int ud = 0; ud < UD; ++ud) {
            const int64_t dpb = db + NWV * ud;
            if (dpb >= npb_dn_valid)
                continue;
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = rbase + mt * 16 + (lane >> 4) * 4 + i;
                        if (row < M)
                            pslice[(int64_t)row * npc + dpb * 32 + half * 16 + (lane & 15)] =
                                acc[ud][half][mt][i];
                    }
        }
    }
}

// Rows per group and slice width.  A wave's gate/up accumulators hold G x
// MT tiles of each half (8 G MT registers) and a K step loads 2 G weight
// pieces and MT activation fragments (4 registers each): G = 8 for one row
// tile, 4 above, keeps a wave within 200 registers.  Wider slices would
// write fewer partial rows of y (slices x M x d x 4 bytes in all); more rows
// per group mean fewer groups, each streaming all the weights once.
FusedPlan plan_fused(const GemmArgs& up, const GemmArgs& dn)
{
    FusedPlan p;
    int64_t mt = ceil_div(up.M, 16);
    p.mt = (int)(mt > 4 ? 4 : (mt < 1 ? 1 : mt));
    p.g = p.mt == 1 ? 8 : 4;
    p.slices = ceil_div(up.geom.npb_valid, p.g);
    p.row_groups = ceil_div(up.M, 16 * p.mt);
    (void)dn;
    return p;
}

size_t fused_partial_bytes(const GemmArgs& dn, const FusedPlan& p)
{
    return (size_t)p.slices * (size_t)dn.M * (size_t)(dn.geom.npb * 32) * sizeof(float);
}

template <int MT, int G>
static void go_fused(const GemmArgs& up, const GemmArgs& dn, const FusedPlan& p, float* partial,
                     hipStream_t s)
{
    constexpr int U = 1;
    constexpr int UD = MT >= 3 ? 2 : 4;
    dim3 grid((unsigned)p.slices, 1u, (unsigned)p.row_groups);
    mlp_fused_kernel<MT, G, U, UD><<<grid, dim3(FU_WAVES * 64), 0, s>>>(
        (const uint16_t*)up.a, up.lda, up.geom.K, (const i32x4*)up.w, up.geom.nkc, up.geom.npb,
        (const i32x4*)dn.w, dn.geom.nkc, dn.geom.npb_valid, partial, dn.geom.npb * 32, (int)up.M);
}

hipError_t launch_fused(const GemmArgs& up, const GemmArgs& dn, const FusedPlan& p, float* partial,
                        hipStream_t s)
{
    if (up.dt != DT_BF16 || dn.dt != DT_BF16)
        return hipErrorInvalidValue;
    switch (p.mt) {
    case 1: go_fused<1, 8>(up, dn, p, partial, s); break;
    case 2: go_fused<2, 4>(up, dn, p, partial, s); break;
    case 3: go_fused<3, 4>(up, dn, p, partial, s); break;
    default: go_fused<4, 4>(up, dn, p, partial, s); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_splitk_reduce(dn, (int)p.slices, partial, s);
}

}  // namespace swg
