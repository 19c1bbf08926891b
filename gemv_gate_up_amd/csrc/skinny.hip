// skinny.hip -- the few-rows (decode) path: out = epi(A . W), built for up
// to 64 rows (the dispatcher's range for bf16); fp32, FP8 and MXFP4 weights
// use it at any M, 64 rows per row group.
//
// Follows the split-over-the-weights idea of "Où part le temps d'un token"
// (section "Un kernel pour les matrices étroites"): with only a few rows of
// activations the grid is cut along the weights, which are large, not along
// the output, which is small.  Each workgroup owns one to four consecutive
// pair blocks of the packed weights (16 gate + 16 up columns, or 32 down
// columns, each; the fp32 one- and two-row kernel can own half of one) and a
// range of K; its four or eight waves take interleaved K pieces, each lane
// streaming 16-byte nontemporal loads with several in flight.  Partial sums
// of the waves are combined in LDS in a fixed order.  When the pair blocks
// alone do not fill the GPU, K is also split across workgroups and a second
// pass adds the slices in ascending order; no atomics are used, so results are
// reproducible run to run (same section: the authors reject an atomic add
// into the output for that reason).  silu(g) * u is applied once the full
// K sum is known (the second pass or the LDS combine), like the bias of the
// "Affine" operation in "Deux opérations de trop"; a down product adds its
// optional bias and residual at the same point.
//
// bf16 weights are multiplied on v_mfma_f32_16x16x32_bf16 with the
// activations as the 16-row A operand: at M <= 16 the matrix unit has spare
// throughput, and above M = 4 plain fp32 FMA on the VALU would take longer
// than streaming the weights.  fp32 weights use VALU FMA at one and two
// rows and v_mfma_f32_16x16x4_f32 from three rows on.
//
// FP8 weights (WF = WF_FP8) halve the streamed bytes: each 16-byte load
// brings 16 E4M3 codes that widen exactly to bf16 (every E4M3 value is a
// bf16 value) with gfx950's packed conversion, feeding two MFMAs over two
// 32-K chunks; the per-column scale multiplies the finished fp32 sum.
// MXFP4 weights (WF_MXFP4) quarter them: 32 E2M1 codes per load feed four
// MFMAs, one per 32-K chunk, and since each chunk of a column is one MX
// block its power-of-two scale is applied by the same conversion (exact).
#include <string.h>

#include "device_common.h"
#include "launch.h"

namespace swg {

constexpr int SK_WAVES = 4;
constexpr int SK_THREADS = SK_WAVES * 64;

constexpr int WF_BF16 = 0, WF_FP8 = 1, WF_MXFP4 = 2;

// Eight E2M1 codes (one dword, low nibble first) times 2^s -> eight bf16
// values in the same order; exact (sc = 2^s, a normal fp32 number).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(int w, float sc) {
    i32x4 r;
    r.x = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    r.y = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    r.z = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    r.w = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    return __builtin_bit_cast(bf16x8, r);
}

// E8M0 scale code (1..254 here) -> 2^(code - 127) as fp32.
__device__ __forceinline__ float e8m0_scale(uint32_t code) {
    return __builtin_bit_cast(float, code << 23);
}

// Eight E4M3 codes (two dwords, lowest byte first) -> eight bf16 values in
// the same order; exact.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(int lo, int hi) {
    i32x4 r;
    r.x = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    r.y = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    r.z = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    r.w = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------- bf16 (MFMA)
// Each wave covers NPB consecutive pair blocks, so one activation fragment
// (MT 16-row tiles of x over a 32-K chunk) feeds 2*NPB*MT MFMAs; with 16 or
// more rows, re-reading that fragment per pair block would cost half as many
// bytes again as the weights.  FP8 and MXFP4 pieces span two and four
// chunks (CH), so each step loads CH activation fragments per row tile.
template <int MT, int U, int NPB, int EPI, bool SPLIT, typename OutT, int WF, int NWV>
__global__ void __launch_bounds__(NWV * 64)
skinny_bf16_kernel(const uint16_t* __restrict__ a, int64_t lda, int64_t kvalid,
                   const i32x4* __restrict__ w, int64_t nkc, int64_t cps,
                   OutT* __restrict__ out, int64_t ldo, int64_t ncols_out,
                   float* __restrict__ partial, int64_t npc, int M,
                   const void* __restrict__ scales, const OutT* __restrict__ resid, int64_t ldr,
                   const OutT* __restrict__ bias)
{
    constexpr bool W8 = WF == WF_FP8;
    constexpr int CH = WF == WF_BF16 ? 1 : (WF == WF_FP8 ? 2 : 4);   // 32-K chunks per piece
    // Software pipelining (below) for bf16 weights and one row tile, where
    // it was measured faster: 8B-class decode at 1, 4, 8 and 16 rows
    // 37.45, 38.3, 39.2, 38.4 -> 37.3, 37.8, 38.6, 37.6 us (with the pieces
    // in flight re-tuned for it in pick_mt_bf16); slower with FP8 or MXFP4
    // weights (8B decode at 16 rows 23.6 -> 25.4 us and 15.6 -> 16.2 us, at
    // one row 20.8 -> 21.7 us and 13.1 -> 14.7 us, also with two pieces in
    // flight) and with four row tiles (0.5B-class MLP at 64 rows 19.8 ->
    // 20.0 us).
    constexpr bool PIPE = WF == WF_BF16 && MT == 1;
    const float* colscale = (const float*)scales;                       // FP8: per column
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t pb0 = (int64_t)blockIdx.x * NPB;
    const int s = blockIdx.y;
    const int rbase = blockIdx.z * 16 * MT;
    const int64_t kbeg = (int64_t)s * cps;
    const int64_t kend = kbeg + cps < nkc ? kbeg + cps : nkc;
    const i32x4* wp = w + pb0 * nkc * 2 * PIECE_VECS + lane;
    // MXFP4: 16 dwords of block scales per piece; lane l reads its column's
    const uint32_t* blkscale =
        WF == WF_MXFP4 ? (const uint32_t*)scales + pb0 * nkc * 2 * 16 + (lane & 15) : nullptr;

    // A operand of lane l: row l % 16 of each 16-row tile, k-group l / 16.
    const int arow = lane & 15;
    const int akoff = (lane >> 4) * 8;

    f32x4 accg[NPB][MT], accu[NPB][MT];
#pragma unroll
    for (int p = 0; p < NPB; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            accg[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // One step of a wave: U pieces per half of each of its NPB pair blocks
    // (K chunks kb, kb + NWV, ...) and the matching activation fragments.
    struct Step {
        i32x4 wg[NPB][U], wu[NPB][U];
        uint32_t sgb[WF == WF_MXFP4 ? NPB : 1][U], sub[WF == WF_MXFP4 ? NPB : 1][U];
        i32x4 xa[U][CH][MT];
    };
    auto issue = [&](int64_t kb, Step& L) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kc = kb + NWV * u;
#pragma unroll
            for (int p = 0; p < NPB; ++p) {
                if (kc < kend) {
                    L.wg[p][u] = load_nt16(wp + (p * nkc * 2 + kc * 2) * PIECE_VECS);
                    L.wu[p][u] = load_nt16(wp + (p * nkc * 2 + kc * 2 + 1) * PIECE_VECS);
                    if constexpr (WF == WF_MXFP4) {
                        L.sgb[p][u] = blkscale[(p * nkc * 2 + kc * 2) * 16];
                        L.sub[p][u] = blkscale[(p * nkc * 2 + kc * 2 + 1) * 16];
                    }
                } else {
                    L.wg[p][u] = i32x4{0, 0, 0, 0};
                    L.wu[p][u] = i32x4{0, 0, 0, 0};
                    if constexpr (WF == WF_MXFP4) {
                        L.sgb[p][u] = 127u * 0x01010101u;   // scale 1 for the zero padding
                        L.sub[p][u] = 127u * 0x01010101u;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kc = kb + NWV * u;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
                const int64_t k = (kc * CH + ch) * 32 + akoff;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row = rbase + mt * 16 + arow;
                    if (kc < kend && row < M && k < kvalid)
                        L.xa[u][ch][mt] = *(const i32x4*)(a + (int64_t)row * lda + k);
                    else
                        L.xa[u][ch][mt] = i32x4{0, 0, 0, 0};
                }
            }
        }
    };
    auto consume = [&](const Step& L) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int p = 0; p < NPB; ++p) {
#pragma unroll
                for (int ch = 0; ch < CH; ++ch) {
                    bf16x8 bg, bu;
                    if constexpr (WF == WF_MXFP4) {
                        bg = e2m1x8_to_bf16(L.wg[p][u][ch], e8m0_scale((L.sgb[p][u] >> (8 * ch)) & 255u));
                        bu = e2m1x8_to_bf16(L.wu[p][u][ch], e8m0_scale((L.sub[p][u] >> (8 * ch)) & 255u));
                    } else if constexpr (W8) {
                        bg = ch == 0 ? e4m3x8_to_bf16(L.wg[p][u].x, L.wg[p][u].y)
                                     : e4m3x8_to_bf16(L.wg[p][u].z, L.wg[p][u].w);
                        bu = ch == 0 ? e4m3x8_to_bf16(L.wu[p][u].x, L.wu[p][u].y)
                                     : e4m3x8_to_bf16(L.wu[p][u].z, L.wu[p][u].w);
                    } else {
                        bg = __builtin_bit_cast(bf16x8, L.wg[p][u]);
                        bu = __builtin_bit_cast(bf16x8, L.wu[p][u]);
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const bf16x8 av = __builtin_bit_cast(bf16x8, L.xa[u][ch][mt]);
                        accg[p][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bg, accg[p][mt],
                                                                               0, 0, 0);
                        accu[p][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bu, accu[p][mt],
                                                                               0, 0, 0);
                    }
                }
            }
        }
    };
    constexpr int64_t STEP = NWV * U;
    if constexpr (PIPE) {
        // two register sets: a step's loads are issued before the MFMAs of
        // the step before it, so the wave always has loads in flight
        Step L0, L1;
        int64_t kb = kbeg + wave;
        if (kb < kend)
            issue(kb, L0);
        for (; kb < kend; kb += 2 * STEP) {
            if (kb + STEP < kend)
                issue(kb + STEP, L1);
            consume(L0);
            if (kb + STEP >= kend)
                break;
            if (kb + 2 * STEP < kend)
                issue(kb + 2 * STEP, L0);
            consume(L1);
        }
    } else {
        for (int64_t kb = kbeg + wave; kb < kend; kb += STEP) {
            Step L;
            issue(kb, L);
            consume(L);
        }
    }

    // Combine the waves in LDS, in wave order, one pair block at a time;
    // the first 256 threads each finish one (row, column) of the 16 x 16
    // tiles.  MFMA result layout: lane l holds rows 4*(l/16) + i (i = 0..3)
    // of column l % 16.
    __shared__ float red[NWV][MT][2][64 * 4];
    const int t = threadIdx.x;
    const int r = t >> 4, c = t & 15;
    const int src = ((r >> 2) * 16 + c) * 4 + (r & 3);
#pragma unroll
    for (int p = 0; p < NPB; ++p) {
        const int64_t pb = pb0 + p;
        if (p > 0)
            __syncthreads();   // the previous pair block's sums have been read
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[wave][mt][0][lane * 4 + i] = accg[p][mt][i];
                red[wave][mt][1][lane * 4 + i] = accu[p][mt][i];
            }
        }
        __syncthreads();
        if (NWV > 4 && t >= 256)
            continue;   // no combining work; the next pair block's barrier is reached
        // column scales of the FP8 weights: entry 32 * pb + 16 * half + c
        const float gs = W8 ? colscale[pb * 32 + c] : 1.f;
        const float us = W8 ? colscale[pb * 32 + 16 + c] : 1.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int wv = 0; wv < NWV; ++wv) {
                g += red[wv][mt][0][src];
                u += red[wv][mt][1][src];
            }
            if (W8) {
                g *= gs;
                u *= us;
            }
            const int row = rbase + mt * 16 + r;
            if (row >= M)
                continue;
            if (SPLIT) {
                float* pr = partial + ((int64_t)s * M + row) * npc + pb * 32;
                pr[c] = g;
                pr[16 + c] = u;
            } else if (EPI == EPI_SWIGLU) {
                const int64_t n = pb * 16 + c;
                if (n < ncols_out)
                    store_out(out + (int64_t)row * ldo + n, silu(g) * u);
            } else {
                const int64_t j = pb * 32 + c;
                if (j < ncols_out)
                    store_out(out + (int64_t)row * ldo + j, plain_tail(g, resid, ldr, bias, row, j));
                if (j + 16 < ncols_out)
                    store_out(out + (int64_t)row * ldo + j + 16,
                              plain_tail(u, resid, ldr, bias, row, j + 16));
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 (matrix)
// fp32 on the matrix unit, v_mfma_f32_16x16x4_f32, from the fp32 piece
// layout: lane l holds column l % 16 and the four consecutive K values
// 4 (l / 16) .. 4 (l / 16) + 3 of the piece's 16.  MFMA j takes K value
// 4 (l / 16) + j as its k index l / 16 for both operands, so the four MFMAs
// of a piece sum all 16, and one 16-byte activation load per lane and row
// tile (row l % 16, the same four K values) feeds them.  Same decomposition,
// combine and epilogue as skinny_bf16_kernel; the VALU kernel below keeps
// one row, where a 16-row MFMA would waste most of its work.
template <int MT, int U, int NPB, int EPI, bool SPLIT, int NWV>
__global__ void __launch_bounds__(NWV * 64)
skinny_f32m_kernel(const float* __restrict__ a, int64_t lda, int64_t kvalid,
                   const f32x4* __restrict__ w, int64_t nkc, int64_t cps,
                   float* __restrict__ out, int64_t ldo, int64_t ncols_out,
                   float* __restrict__ partial, int64_t npc, int M,
                   const float* __restrict__ resid, int64_t ldr, const float* __restrict__ bias)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t pb0 = (int64_t)blockIdx.x * NPB;
    const int s = blockIdx.y;
    const int rbase = blockIdx.z * 16 * MT;
    const int64_t kbeg = (int64_t)s * cps;
    const int64_t kend = kbeg + cps < nkc ? kbeg + cps : nkc;
    const f32x4* wp = w + pb0 * nkc * 2 * PIECE_VECS + lane;
    const int arow = lane & 15;
    const int akoff = (lane >> 4) * 4;

    f32x4 accg[NPB][MT], accu[NPB][MT];
#pragma unroll
    for (int p = 0; p < NPB; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            accg[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    for (int64_t kb = kbeg + wave; kb < kend; kb += NWV * U) {
        f32x4 wg[NPB][U], wu[NPB][U], xa[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kc = kb + NWV * u;
#pragma unroll
            for (int p = 0; p < NPB; ++p) {
                if (kc < kend) {
                    wg[p][u] = __builtin_nontemporal_load(wp + (p * nkc * 2 + kc * 2) * PIECE_VECS);
                    wu[p][u] = __builtin_nontemporal_load(wp + (p * nkc * 2 + kc * 2 + 1) * PIECE_VECS);
                } else {
                    wg[p][u] = f32x4{0.f, 0.f, 0.f, 0.f};
                    wu[p][u] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kc = kb + NWV * u;
            const int64_t k = kc * 16 + akoff;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = rbase + mt * 16 + arow;
                xa[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (kc < kend && row < M && k < kvalid)
                    xa[u][mt] = *(const f32x4*)(a + (int64_t)row * lda + k);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int p = 0; p < NPB; ++p)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        accg[p][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            xa[u][mt][j], wg[p][u][j], accg[p][mt], 0, 0, 0);
                        accu[p][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            xa[u][mt][j], wu[p][u][j], accu[p][mt], 0, 0, 0);
                    }
    }

    // Combine the waves in LDS, in wave order, as skinny_bf16_kernel does;
    // lane l holds rows 4 (l / 16) + i (i = 0..3) of column l % 16.
    __shared__ float red[NWV][MT][2][64 * 4];
    const int t = threadIdx.x;
    const int r = t >> 4, c = t & 15;
    const int src = ((r >> 2) * 16 + c) * 4 + (r & 3);
#pragma unroll
    for (int p = 0; p < NPB; ++p) {
        const int64_t pb = pb0 + p;
        if (p > 0)
            __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[wave][mt][0][lane * 4 + i] = accg[p][mt][i];
                red[wave][mt][1][lane * 4 + i] = accu[p][mt][i];
            }
        }
        __syncthreads();
        if (NWV > 4 && t >= 256)
            continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int wv = 0; wv < NWV; ++wv) {
                g += red[wv][mt][0][src];
                u += red[wv][mt][1][src];
            }
            const int row = rbase + mt * 16 + r;
            if (row >= M)
                continue;
            if (SPLIT) {
                float* pr = partial + ((int64_t)s * M + row) * npc + pb * 32;
                pr[c] = g;
                pr[16 + c] = u;
            } else if (EPI == EPI_SWIGLU) {
                const int64_t n = pb * 16 + c;
                if (n < ncols_out)
                    store_out(out + (int64_t)row * ldo + n, silu(g) * u);
            } else {
                const int64_t j = pb * 32 + c;
                if (j < ncols_out)
                    store_out(out + (int64_t)row * ldo + j, plain_tail(g, resid, ldr, bias, row, j));
                if (j + 16 < ncols_out)
                    store_out(out + (int64_t)row * ldo + j + 16,
                              plain_tail(u, resid, ldr, bias, row, j + 16));
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 (VALU)
// A workgroup covers 16 / CS columns of each half of one pair block (CS
// workgroups share a pair block; CS > 1 only without a split of K).  Lane l
// covers column l % CW of that share, k-group (l / CW) % 4 (4 consecutive K
// values) and piece CS * v + l / (4 CW) of its step v, so every lane's
// 16-byte load is useful; the lanes of a column are added with butterfly
// steps whose result is the same in each of them, then the waves are added
// in LDS.  With CS = 1 a lane covers column l % 16 and k-group l / 16 of
// every piece.
template <int RT, int U, int EPI, bool SPLIT, typename OutT, int CS = 1>
__global__ void __launch_bounds__(SK_THREADS)
skinny_f32_kernel(const float* __restrict__ a, int64_t lda, int64_t kvalid,
                  const f32x4* __restrict__ w, int64_t nkc, int64_t cps,
                  OutT* __restrict__ out, int64_t ldo, int64_t ncols_out,
                  float* __restrict__ partial, int64_t npc, int M,
                  const OutT* __restrict__ resid, int64_t ldr, const OutT* __restrict__ bias)
{
    static_assert(CS == 1 || ((CS == 2 || CS == 4) && !SPLIT), "column shares without a K split");
    constexpr int CW = 16 / CS;   // columns of each half per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t pb = blockIdx.x / CS;
    const int cbase = (int)(blockIdx.x % CS) * CW;
    const int s = blockIdx.y;
    const int rbase = blockIdx.z * RT;
    const int64_t kbeg = (int64_t)s * cps;
    const int64_t kend = kbeg + cps < nkc ? kbeg + cps : nkc;
    const int lp = lane / (4 * CW);   // piece of the lane within a step's CS pieces
    const int kgrp = (lane / CW) % 4;
    const f32x4* wp = w + pb * nkc * 2 * PIECE_VECS + kgrp * 16 + cbase + lane % CW;
    const int koff = kgrp * 4;

    float accg[RT], accu[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        accg[r] = 0.f;
        accu[r] = 0.f;
    }

    // step v of the loop covers pieces kbeg + CS * v .. + CS - 1
    const int64_t nv = (kend - kbeg + CS - 1) / CS;
    for (int64_t vb = wave; vb < nv; vb += SK_WAVES * U) {
        f32x4 wg[U], wu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kc = kbeg + (vb + SK_WAVES * u) * CS + lp;
            if (kc < kend) {
                wg[u] = __builtin_nontemporal_load(wp + (kc * 2) * PIECE_VECS);
                wu[u] = __builtin_nontemporal_load(wp + (kc * 2 + 1) * PIECE_VECS);
            } else {
                wg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                wu[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        // The activation vectors are loaded before any of them is used:
        // every piece's at once when they fit in a few registers (the
        // one-row decode: 8 loads in flight instead of 8 round trips one
        // after another), else a piece's rows at once.  The FMAs keep their
        // order.
        constexpr int XB = U * RT <= 16 ? U : 1;   // pieces whose vectors are loaded together
#pragma unroll
        for (int u0 = 0; u0 < U; u0 += XB) {
            f32x4 xv[XB][RT];
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int64_t kc = kbeg + (vb + SK_WAVES * (u0 + i)) * CS + lp;
                const int64_t k = kc * 16 + koff;
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const int row = rbase + r;
                    xv[i][r] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (row < M && kc < kend && k < kvalid)
                        xv[i][r] = *(const f32x4*)(a + (int64_t)row * lda + k);
                }
            }
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int u = u0 + i;
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    if (rbase + r < M) {   // uniform across the wave
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            accg[r] = __builtin_fmaf(xv[i][r][e], wg[u][e], accg[r]);
                            accu[r] = __builtin_fmaf(xv[i][r][e], wu[u][e], accu[r]);
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int m = CW; m < 64; m *= 2) {
            accg[r] += __shfl_xor(accg[r], m);
            accu[r] += __shfl_xor(accu[r], m);
        }
    }
    __shared__ float red[SK_WAVES][2][RT][CW];
    if (lane < CW) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            red[wave][0][r][lane] = accg[r];
            red[wave][1][r][lane] = accu[r];
        }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t >= RT * CW)
        return;
    const int r = t / CW, c = cbase + t % CW;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int wv = 0; wv < SK_WAVES; ++wv) {
        g += red[wv][0][r][t % CW];
        u += red[wv][1][r][t % CW];
    }
    const int row = rbase + r;
    if (row >= M)
        return;
    if (SPLIT) {
        float* pr = partial + ((int64_t)s * M + row) * npc + pb * 32;
        pr[c] = g;
        pr[16 + c] = u;
    } else if (EPI == EPI_SWIGLU) {
        const int64_t n = pb * 16 + c;
        if (n < ncols_out)
            store_out(out + (int64_t)row * ldo + n, silu(g) * u);
    } else {
        const int64_t j = pb * 32 + c;
        if (j < ncols_out)
            store_out(out + (int64_t)row * ldo + j, plain_tail(g, resid, ldr, bias, row, j));
        if (j + 16 < ncols_out)
            store_out(out + (int64_t)row * ldo + j + 16,
                      plain_tail(u, resid, ldr, bias, row, j + 16));
    }
}

// ---------------------------------------------------------------- second pass
// Adds the K slices in ascending slice order, then applies the epilogue.
// The slices are loaded eight at a time before they are added, so a thread
// waits for one memory round trip per eight slices rather than per slice;
// the additions keep their order (a slice past S adds nothing, not +0).
constexpr int RED_BATCH = 8;

template <int EPI, typename OutT>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ partial, int S, int M, int64_t npc,
                     OutT* __restrict__ out, int64_t ldo, int64_t ncols_out, int col_blocks,
                     const OutT* __restrict__ resid, int64_t ldr, const OutT* __restrict__ bias)
{
    const int row = blockIdx.x / col_blocks;
    const int64_t col = (int64_t)(blockIdx.x % col_blocks) * 256 + threadIdx.x;
    if (col >= ncols_out)
        return;
    const int64_t slice = (int64_t)M * npc;   // floats per slice
    if (EPI == EPI_SWIGLU) {
        const float* pr = partial + (int64_t)row * npc + (col / 16) * 32 + (col % 16);
        float g = 0.f, u = 0.f;
        for (int s0 = 0; s0 < S; s0 += RED_BATCH) {
            float tg[RED_BATCH], tu[RED_BATCH];
#pragma unroll
            for (int j = 0; j < RED_BATCH; ++j) {
                tg[j] = s0 + j < S ? pr[(s0 + j) * slice] : 0.f;
                tu[j] = s0 + j < S ? pr[(s0 + j) * slice + 16] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < RED_BATCH; ++j) {
                if (s0 + j < S) {
                    g += tg[j];
                    u += tu[j];
                }
            }
        }
        store_out(out + (int64_t)row * ldo + col, silu(g) * u);
    } else {
        const float* pr = partial + (int64_t)row * npc + col;
        float v = 0.f;
        for (int s0 = 0; s0 < S; s0 += RED_BATCH) {
            float t[RED_BATCH];
#pragma unroll
            for (int j = 0; j < RED_BATCH; ++j)
                t[j] = s0 + j < S ? pr[(s0 + j) * slice] : 0.f;
#pragma unroll
            for (int j = 0; j < RED_BATCH; ++j)
                if (s0 + j < S)
                    v += t[j];
        }
        store_out(out + (int64_t)row * ldo + col, plain_tail(v, resid, ldr, bias, row, col));
    }
}

// ---------------------------------------------------------------- planning
// fp32 calls of at least this many rows take the matrix-unit kernel
// (skinny_f32m_kernel), fewer the VALU kernel.  8B-class shape, VALU ->
// matrix unit: 2 rows 78.5-78.8 -> 78.9-79.4 us; 4, 8, 16 and 64 rows 88,
// 142, 201, 691 -> 80-81, 85, 93-94, 227 us (the VALU kernel reads each
// activation vector once per row and lane); 0.5B-class at 4 and 16 rows
// 13.3, 22.7 -> 11.7, 13.5 us.
constexpr int64_t F32_MFMA_MIN_M = 3;

static int bf16_row_tiles(int64_t M) {
    int64_t mt = ceil_div(M, 16);
    return (int)(mt > 4 ? 4 : (mt < 1 ? 1 : mt));
}

// Pair blocks per wave of the bf16 kernel with bf16 weights: two once x's
// fragment is as large as a weight piece (more than 8 rows), one otherwise.
// pick_mt_bf16 overrides it for some gate/up products of 3 to 16 rows (two
// or four), and for FP8 and MXFP4 weights sets the count by row range and
// product (FP8 planned as two).
static int bf16_pair_blocks(int64_t M, int dt) {
    return (dt == DT_FP8W || M > 8) ? 2 : 1;
}

// Rows per workgroup of the fp32 VALU kernel, which serves one and two rows.
static int f32_row_tile(int64_t M) {
    return M >= 2 ? 2 : 1;
}

SkinnyPlan plan_skinny(const GemmArgs& g, int num_cus)
{
    SkinnyPlan p;
    p.grid_pb = ceil_div(g.ncols_out, g.geom.cols_per_pb);
    p.pb_per_wg = g.dt != DT_F32 ? bf16_pair_blocks(g.M, g.dt) : 1;
    if (g.dt != DT_F32 && g.epi == EPI_PLAIN && g.M > 16)
        p.pb_per_wg = 1;
    const bool f32m = g.dt == DT_F32 && g.M >= F32_MFMA_MIN_M;
    p.row_tile = (g.dt != DT_F32 || f32m) ? 16 * bf16_row_tiles(g.M) : f32_row_tile(g.M);
    p.row_groups = ceil_div(g.M, p.row_tile);
    // Split K only when there are too few pair blocks (units of weight
    // streaming) to keep every CU busy; two pair blocks per workgroup are
    // still two units of work.  A gate/up product over more than 16 rows
    // carries several row tiles of matrix work per pair block and its
    // partials grow with M: one pair block per CU is enough there (the
    // 0.5B-class MLP at 64 rows: 14.1 us with a 2-way split and its second
    // pass, 11.1 us without).
    const int64_t base = p.grid_pb * p.row_groups;
    const int64_t target =
        (g.epi == EPI_SWIGLU && p.row_tile > 16) ? (int64_t)num_cus : 2 * (int64_t)num_cus;
    // each slice streams at least 16 pieces (the 0.5B-class MLP's down
    // product at 64 rows: 19 pieces per slice 11.9 us, 9.5 pieces 13.5 us)
    const int64_t min_chunks = 16;
    // A split costs a second launch of a few microseconds: not worth it when
    // each pair block streams little (the tiny fp32 decode, 64 KB per pair
    // block: 7.1 us with a 4-way split and its second pass, 5.1 us without).
    const bool small = g.geom.bytes() < (int64_t)128 * 1024 * p.grid_pb;
    int64_t S = 1;
    while (!small && base * S < target && g.geom.nkc / (2 * S) >= min_chunks && S < 64)
        S *= 2;
    p.chunks_per_split = ceil_div(g.geom.nkc, S);
    p.splits = (int)ceil_div(g.geom.nkc, p.chunks_per_split);
    return p;
}

size_t skinny_partial_bytes(const GemmArgs& g, const SkinnyPlan& p)
{
    if (p.splits <= 1)
        return 0;
    return (size_t)p.splits * (size_t)g.M * (size_t)(g.geom.npb * 32) * sizeof(float);
}

template <int MT, int U, int NPB, int EPI, bool SPLIT, typename OutT, int WF, int NWV>
static void go_bf16(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    // With two pair blocks per workgroup and an odd count, the last
    // workgroup's second pair block is padding (zero weights, never stored):
    // the packed buffer holds a multiple of 8 pair blocks.
    dim3 grid((unsigned)ceil_div(p.grid_pb, NPB), (unsigned)p.splits, (unsigned)p.row_groups);
    const void* scales = WF != WF_BF16 ? (const uint8_t*)g.w + g.geom.scale_offset() : nullptr;
    skinny_bf16_kernel<MT, U, NPB, EPI, SPLIT, OutT, WF, NWV><<<grid, dim3(NWV * 64), 0, s>>>(
        (const uint16_t*)g.a, g.lda, g.geom.K, (const i32x4*)g.w, g.geom.nkc, p.chunks_per_split,
        (OutT*)g.out, g.ldo, g.ncols_out, partial, g.geom.npb * 32, (int)g.M, scales,
        (const OutT*)g.resid, g.ldr, (const OutT*)g.bias);
}

template <int MT, int U, int NPB, int EPI, int WF, int NWV = SK_WAVES>
static void pick_split_bf16(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    if (p.splits > 1)
        go_bf16<MT, U, NPB, EPI, true, uint16_t, WF, NWV>(g, p, partial, s);
    else
        go_bf16<MT, U, NPB, EPI, false, uint16_t, WF, NWV>(g, p, partial, s);
}

// Loads in flight per lane: 2*NPB*U weight pieces plus U*MT activation
// fragments (times two with FP8 weights), measured on the 8B- and
// 72B-class decode shapes.
constexpr int64_t MXFP4_WIDE_PB_CUS = 256;   // MI355X compute units
constexpr int64_t SKINNY_CUS = 256;          // the same, for the bf16 shape choices

template <int EPI, int WF>
static void pick_mt_bf16(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    // FP8 and MXFP4 pieces already span 64 and 128 K: fewer in flight; the
    // MXFP4 activation fragments (4 per piece and row tile) bound U above
    // two row tiles
    constexpr bool Q = WF != WF_BF16;
    // Above 8 rows a gate/up product takes four pair blocks per workgroup
    // (one activation fragment feeds more weights) unless two leave the
    // busiest CU less to stream: its workgroups times each one's bytes,
    // counted in quarters of a bf16 pair block (a bf16 pair block 4, FP8
    // 2, MXFP4 1; one 16-row activation tile over the same K 2).  A small
    // product takes two (the 0.5B-class shape, 304 pair blocks: at 16 rows
    // bf16 9.0 -> 6.5 us, its MLP 16.7 -> 14.1 us, FP8 7.2 -> 5.3 us, MXFP4
    // 6.1 -> 4.7 us), and so does one whose four-block grid would leave a
    // few CUs with a second workgroup or half of them idle (7B-class 3584 x
    // 18944 at 16 rows, 296 workgroups: bf16 56.5 -> 48.9 us, FP8 31.9 ->
    // 28.9 us; 3B-class 3072 x 8192, 128 workgroups: 16 rows bf16 23.3 ->
    // 18.8 us, MXFP4 11.4 -> 8.6 us, 64 rows bf16 35.1 -> 26.9 us; 1B-class
    // 2048 x 8192 at 16 rows 16.7 -> 13.5 us).  The 8B- and 72B-class
    // shapes keep four.
    const int64_t wq = WF == WF_BF16 ? 4 : (WF == WF_FP8 ? 2 : 1);
    const int64_t xq = 2 * (p.row_tile / 16);
    auto cu_load = [&](int64_t n) {
        return ceil_div(ceil_div(p.grid_pb, n) * p.splits, SKINNY_CUS) * (wq * n + xq);
    };
    const bool few4 = EPI == EPI_SWIGLU && cu_load(4) > cu_load(2);
    // Likewise up to 8 rows with FP8 and MXFP4 weights: where two pair
    // blocks per workgroup would give fewer workgroups than CUs, one (the
    // 0.5B-class shape at 1, 4 and 8 rows: MXFP4 4.1, 4.2, 4.7 -> 3.9,
    // 4.05, 4.3 us; FP8 at 4 and 8 rows 5.4, 5.6 -> 4.7, 5.0 us; the 8B-
    // and 72B-class shapes unchanged).
    const bool few2 = EPI == EPI_SWIGLU && ceil_div(p.grid_pb, 2) * p.splits < SKINNY_CUS;
    // Where two pair blocks per workgroup give exactly one workgroup per CU
    // (512 pair blocks: d_ff = 8192), FP8 and MXFP4 gate/up products of 3
    // to 8 rows run them on eight waves, one piece per half in flight: four
    // waves would leave one wave per SIMD with nothing to hide its loads
    // behind (3B-class 3072 x 8192: FP8 at 4 and 8 rows 12.8, 13.35 ->
    // 10.2, 10.95 us, MXFP4 at 8 rows 10.0 -> 8.2 us; with more than one
    // workgroup per CU four waves stay faster: 8B-, 13B- and 72B-class FP8
    // at 8 rows 2-5% slower on eight).
    const bool one2 = EPI == EPI_SWIGLU && ceil_div(p.grid_pb, 2) * p.splits <= SKINNY_CUS;
    const bool wide4 = EPI == EPI_SWIGLU && !few4;   // gate/up products at 17-64 rows (below)
    switch (p.row_tile / 16) {
    case 1:
        if constexpr (WF == WF_MXFP4) {
            // one piece in flight per half; above 8 rows, four pair blocks
            // per wave when that still leaves a workgroup per CU (measured
            // at 1, 8 and 16 rows on the 8B and 72B shapes); up to 4 rows,
            // eight waves per workgroup (8B decode at one row 14.1 -> 13.3
            // us, 72B 45.0 -> 44.0 us; slower at 8 rows on the 8B shape),
            // and so does a down product above 8 rows (the 72B-class MLP at
            // 16 rows 91.5 -> 84.2 us; an 8B-class gate/up product at 16
            // rows is slower with eight: 15.7 -> 16.9 us).  Above 8 rows each
            // workgroup reads as many activation bytes as it has K, so the
            // smaller gate/up products also take four pair blocks per wave,
            // on eight waves (8B-class at 16 rows 15.8 -> 15.5 us)
            if (g.M > 8 && !few4 && p.grid_pb >= 4 * MXFP4_WIDE_PB_CUS)
                pick_split_bf16<1, 1, 4, EPI, WF>(g, p, partial, s);
            else if (g.M > 8 && few4)
                pick_split_bf16<1, 1, 2, EPI, WF, 8>(g, p, partial, s);
            else if (g.M > 8 && EPI == EPI_SWIGLU)
                pick_split_bf16<1, 1, 4, EPI, WF, 8>(g, p, partial, s);
            else if (g.M <= 4 && few2)
                pick_split_bf16<1, 1, 1, EPI, WF, 8>(g, p, partial, s);
            else if (g.M <= 4 || (EPI == EPI_PLAIN && g.M > 8))
                pick_split_bf16<1, 1, 2, EPI, WF, 8>(g, p, partial, s);
            else if (few2)
                pick_split_bf16<1, 1, 1, EPI, WF, 8>(g, p, partial, s);
            else if (one2)
                pick_split_bf16<1, 1, 2, EPI, WF, 8>(g, p, partial, s);
            else
                pick_split_bf16<1, 1, 2, EPI, WF>(g, p, partial, s);
        } else if constexpr (Q) {
            // FP8: up to 2 rows, eight waves per workgroup (8B decode at one
            // row 21.4 -> 21.0 us, two rows 21.1 -> 20.9 us; at four rows
            // 21.0 -> 21.4 us), each on one pair block: twice the
            // workgroups, 3.5 per CU instead of 1.75 (one row 20.87 ->
            // 20.68 us; four pieces per half, four waves, or two pair blocks
            // with one piece: 21.4-22.1 us); a down product above 8 rows also on eight
            // waves, one piece per half in flight (72B-class MLP at 16 rows
            // 130.4 -> 127.4 us); a gate/up product above 8 rows takes four
            // pair blocks per wave on eight waves, one piece per half in
            // flight: each workgroup's activation bytes (its whole K range
            // of 16 rows) then feed twice the weights (8B-class at 16 rows
            // 23.7 -> 23.2 us, 72B-class MLP 124.6 -> 119.8 us)
            if (g.M <= 2)
                pick_split_bf16<1, 2, 1, EPI, WF, 8>(g, p, partial, s);
            else if (EPI == EPI_PLAIN && g.M > 8)
                pick_split_bf16<1, 1, 2, EPI, WF, 8>(g, p, partial, s);
            else if (g.M > 8 && few4)
                pick_split_bf16<1, 1, 2, EPI, WF, 8>(g, p, partial, s);
            else if (g.M > 8)
                pick_split_bf16<1, 1, 4, EPI, WF, 8>(g, p, partial, s);
            else if (few2)
                pick_split_bf16<1, 2, 1, EPI, WF, 8>(g, p, partial, s);
            else if (one2)
                pick_split_bf16<1, 1, 2, EPI, WF, 8>(g, p, partial, s);
            else
                pick_split_bf16<1, 2, 2, EPI, WF>(g, p, partial, s);
        } else {
            // a gate/up product above 8 rows: four pair blocks per wave, so
            // each workgroup's activation bytes (its whole K range of 16
            // rows) feed twice the weights (8B-class at 16 rows 40.1 -> 38.3
            // us, 72B-class MLP at 16 rows 225.7 -> 219.0 us; eight waves, or
            // four pieces in flight, were slower); with the pipelined loop
            // one piece per half and step (38.4 -> 37.6 us; two: 38.4).
            // From three to eight rows, a gate/up product of 2 to 4 pair
            // blocks per CU takes two pair blocks per wave, one piece per
            // half and step (8B-class, 896 pair blocks, at 4 and 8 rows
            // 37.4, 38.2 -> 36.7-36.8, 37.2-37.3 us).  Outside that range it
            // was slower: 304 pair blocks (0.5B-class) 5.8, 6.0 -> 6.9,
            // 6.8 us; 1,848 (72B-class) 143.8, 145.0 -> 145.3, 145.8 us.  At
            // one row it gains nothing, and at 16 rows it is slower (37.2 ->
            // 39.0 us).  Other products above two rows: four pieces per half
            // (8B-class at 4 rows 38.3 -> 37.8 us pipelined; eight there:
            // 38.8); up to two rows eight (37.3 us; four: 38.0)
            if (g.M > 8 && few4)
                pick_split_bf16<1, 2, 2, EPI, WF>(g, p, partial, s);
            else if (g.M > 8 && EPI == EPI_SWIGLU)
                pick_split_bf16<1, 1, 4, EPI, WF>(g, p, partial, s);
            else if (g.M > 2 && EPI == EPI_SWIGLU && p.grid_pb >= 2 * SKINNY_CUS &&
                     p.grid_pb <= 4 * SKINNY_CUS)
                pick_split_bf16<1, 1, 2, EPI, WF>(g, p, partial, s);
            else if (p.pb_per_wg == 2)
                pick_split_bf16<1, 4, 2, EPI, WF>(g, p, partial, s);
            else if (g.M > 2)
                pick_split_bf16<1, 4, 1, EPI, WF>(g, p, partial, s);
            else
                pick_split_bf16<1, 8, 1, EPI, WF>(g, p, partial, s);
        }
        break;
    // above 16 rows a plain (down) product takes one pair block per wave:
    // its few 32-column blocks are better spread over more workgroups; with
    // bf16 weights eight waves share each workgroup's K range, halving the
    // serial load-to-MFMA trips per wave (the 0.5B-class MLP at 64 rows:
    // gate/up 11.0 -> 10.2 us, down 11.8 -> 11.2 us), each with one piece
    // per half in flight: fewer registers (120 instead of 155 at 64 rows)
    // outweigh the extra trip (8B-class gate/up at 32, 48 and 64 rows 52.4,
    // 56.4, 64.4 -> 46.5, 52.5, 60.8 us; 0.5B-class MLP at 64 rows 22.2 ->
    // 21.4 us)
    // A gate/up product of a large matrix takes four pair blocks per
    // workgroup on four waves, one piece in flight: each workgroup reads its
    // whole K range of the 17-64 activation rows, so four halve those reads
    // against two.  bf16: 8B-class at 32, 48, 64 rows 45.4, 52.2, 58.8 ->
    // 40.0, 43.9, 48.4 us; 72B-class at 32 and 64 rows 168, 224 -> 149, 175
    // us (eight waves 1-5% slower).  FP8 weights: 8B-class at 32 and 64
    // rows 32, 48 -> 27.8, 36.7 us, the 72B-class MLP at 32 rows 185 -> 165
    // us; MXFP4: 27, 41 -> 21.6, 32 us, the 72B-class MLP at 64 rows 264 ->
    // 222 us.  A small one keeps two (the 0.5B-class MLP at 64 rows).
    case 2:
        if (wide4)
            pick_split_bf16<2, 1, 4, EPI, WF, 4>(g, p, partial, s);
        else
            pick_split_bf16<2, Q ? 2 : 1, EPI == EPI_PLAIN ? 1 : 2, EPI, WF, Q ? SK_WAVES : 8>(g, p, partial, s);
        break;
    case 3:
        if (wide4)
            pick_split_bf16<3, 1, 4, EPI, WF, 4>(g, p, partial, s);
        else
            pick_split_bf16<3, WF == WF_FP8 ? 2 : 1, EPI == EPI_PLAIN ? 1 : 2, EPI, WF, Q ? SK_WAVES : 8>(g, p, partial, s);
        break;
    default:
        if (wide4)
            pick_split_bf16<4, 1, 4, EPI, WF, 4>(g, p, partial, s);
        else
            pick_split_bf16<4, WF == WF_FP8 ? 2 : 1, EPI == EPI_PLAIN ? 1 : 2, EPI, WF, Q ? SK_WAVES : 8>(g, p, partial, s);
        break;
    }
}

// Workgroups per pair block of the fp32 VALU kernel when the pair blocks
// alone would leave at least half the CUs without a workgroup (no K split):
// two, each lane group still reading whole 128-byte lines (512 x 2048 at
// one row 4.18 -> 4.03-4.28 us, at two rows 4.62 -> 4.42-4.47 us, its MLP
// 9.95 -> 9.85 us); four, with 64-byte segments, were slower (5.5, 6.0,
// 11.0 us).
constexpr int F32_COL_SHARES = 2;

template <int RT, int U, int EPI, bool SPLIT, int CS = 1>
static void go_f32(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    dim3 grid((unsigned)(p.grid_pb * CS), (unsigned)p.splits, (unsigned)p.row_groups);
    skinny_f32_kernel<RT, U, EPI, SPLIT, float, CS><<<grid, dim3(SK_THREADS), 0, s>>>(
        (const float*)g.a, g.lda, g.geom.K, (const f32x4*)g.w, g.geom.nkc, p.chunks_per_split,
        (float*)g.out, g.ldo, g.ncols_out, partial, g.geom.npb * 32, (int)g.M,
        (const float*)g.resid, g.ldr, (const float*)g.bias);
}

template <int RT, int EPI>
static void pick_split_f32(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    if (p.splits > 1)
        go_f32<RT, 8, EPI, true>(g, p, partial, s);
    else if (p.grid_pb * p.row_groups * 2 <= SKINNY_CUS)
        go_f32<RT, 8, EPI, false, F32_COL_SHARES>(g, p, partial, s);
    else
        go_f32<RT, 8, EPI, false>(g, p, partial, s);
}

template <int EPI>
static void pick_rt_f32(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    if (p.row_tile == 1)
        pick_split_f32<1, EPI>(g, p, partial, s);
    else
        pick_split_f32<2, EPI>(g, p, partial, s);
}

template <int MT, int U, int NPB, int EPI, bool SPLIT, int NWV>
static void go_f32m(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    dim3 grid((unsigned)ceil_div(p.grid_pb, NPB), (unsigned)p.splits, (unsigned)p.row_groups);
    skinny_f32m_kernel<MT, U, NPB, EPI, SPLIT, NWV><<<grid, dim3(NWV * 64), 0, s>>>(
        (const float*)g.a, g.lda, g.geom.K, (const f32x4*)g.w, g.geom.nkc, p.chunks_per_split,
        (float*)g.out, g.ldo, g.ncols_out, partial, g.geom.npb * 32, (int)g.M,
        (const float*)g.resid, g.ldr, (const float*)g.bias);
}

template <int MT, int U, int NPB, int EPI, int NWV>
static void pick_split_f32m(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    if (p.splits > 1)
        go_f32m<MT, U, NPB, EPI, true, NWV>(g, p, partial, s);
    else
        go_f32m<MT, U, NPB, EPI, false, NWV>(g, p, partial, s);
}

// Two pair blocks per workgroup, so each activation load feeds twice the
// MFMAs (measured against one: 8B-class at 4, 8, 16 rows 81.5, 86, 93.8 ->
// 77, 77.7, 81 us with two pieces in flight; at 32 and 64 rows 129, 227 ->
// 116.7, 195.7 us; 0.5B-class at 16 rows unchanged, at 64 rows 29.5 ->
// 25.7 us).  The packed buffer holds a multiple of 8 pair blocks, so the
// second one of the last workgroup is zero padding.
template <int EPI>
static void pick_mt_f32m(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    switch (p.row_tile / 16) {
    case 1: pick_split_f32m<1, 2, 2, EPI, 4>(g, p, partial, s); break;
    case 2: pick_split_f32m<2, 1, 2, EPI, 8>(g, p, partial, s); break;
    case 3: pick_split_f32m<3, 1, 2, EPI, 8>(g, p, partial, s); break;
    default: pick_split_f32m<4, 1, 2, EPI, 8>(g, p, partial, s); break;
    }
}

template <int EPI, typename OutT>
static void go_reduce(const GemmArgs& g, const SkinnyPlan& p, const float* partial, hipStream_t s)
{
    const int col_blocks = (int)ceil_div(g.ncols_out, 256);
    splitk_reduce_kernel<EPI, OutT><<<dim3((unsigned)(col_blocks * g.M)), dim3(256), 0, s>>>(
        partial, p.splits, (int)g.M, g.geom.npb * 32, (OutT*)g.out, g.ldo, g.ncols_out,
        col_blocks, (const OutT*)g.resid, g.ldr, (const OutT*)g.bias);
}

hipError_t launch_splitk_reduce(const GemmArgs& g, int splits, const float* partial, hipStream_t s)
{
    SkinnyPlan p;
    memset(&p, 0, sizeof p);
    p.splits = splits;
    if (g.dt != DT_F32) {
        if (g.epi == EPI_SWIGLU)
            go_reduce<EPI_SWIGLU, uint16_t>(g, p, partial, s);
        else
            go_reduce<EPI_PLAIN, uint16_t>(g, p, partial, s);
    } else {
        if (g.epi == EPI_SWIGLU)
            go_reduce<EPI_SWIGLU, float>(g, p, partial, s);
        else
            go_reduce<EPI_PLAIN, float>(g, p, partial, s);
    }
    return hipGetLastError();
}

hipError_t launch_skinny(const GemmArgs& g, const SkinnyPlan& p, float* partial, hipStream_t s)
{
    if (g.dt == DT_BF16) {
        if (g.epi == EPI_SWIGLU)
            pick_mt_bf16<EPI_SWIGLU, WF_BF16>(g, p, partial, s);
        else
            pick_mt_bf16<EPI_PLAIN, WF_BF16>(g, p, partial, s);
    } else if (g.dt == DT_FP8W) {
        if (g.epi == EPI_SWIGLU)
            pick_mt_bf16<EPI_SWIGLU, WF_FP8>(g, p, partial, s);
        else
            pick_mt_bf16<EPI_PLAIN, WF_FP8>(g, p, partial, s);
    } else if (g.dt == DT_MXFP4W) {
        if (g.epi == EPI_SWIGLU)
            pick_mt_bf16<EPI_SWIGLU, WF_MXFP4>(g, p, partial, s);
        else
            pick_mt_bf16<EPI_PLAIN, WF_MXFP4>(g, p, partial, s);
    } else if (g.M >= F32_MFMA_MIN_M) {
        if (g.epi == EPI_SWIGLU)
            pick_mt_f32m<EPI_SWIGLU>(g, p, partial, s);
        else
            pick_mt_f32m<EPI_PLAIN>(g, p, partial, s);
    } else {
        if (g.epi == EPI_SWIGLU)
            pick_rt_f32<EPI_SWIGLU>(g, p, partial, s);
        else
            pick_rt_f32<EPI_PLAIN>(g, p, partial, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits <= 1)
        return e;
    return launch_splitk_reduce(g, p.splits, partial, s);
}

}  // namespace swg
