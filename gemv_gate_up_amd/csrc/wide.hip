// wide.hip -- instantiates the many-rows MFMA GEMM of wide_kernel.h with the
// tile shape and pipeline depth measured best on MI355X.
#include "wide_kernel.h"

namespace swg {

// 256 x 256 fused-column tile, 8 waves (2 per SIMD) of 64 x 128, stages of
// one 32-K chunk, four stages in the LDS ring (up to three in flight); the
// two waves of each SIMD run the ping-pong schedule (one issues a step of
// MFMAs while the other reads fragments and issues loads).  Measured on the
// 8B-class prefill: 0.706-0.708 ms against 0.727-0.733 ms for the
// interleaved schedule of the same tile; a fifth stage, raising the MFMA
// wave's priority, or issuing the loads before the fragment reads did not
// help.
struct WideCfg {
    static constexpr int BM = 256, BN = 256, WGM = 4, WGN = 2, KCS = 1, STAGES = 4;
    static constexpr int GROUP_M = 8;
};

// The two-pass schedule keeps silu(gate) in registers beside the up
// accumulators, so at the same register budget its tile holds half as many
// output columns: 256 rows x 128 outputs, 8 waves of 64 x 64.
struct WidePhasedCfg {
    static constexpr int BM = 256, BN = 128, WGM = 4, WGN = 2, KCS = 1, STAGES = 4;
    static constexpr int GROUP_M = 8;
};
static_assert(WideCfg::BN / 32 == WidePhasedCfg::BN / 16, "both schedules tile 8 pair blocks");

// The last, partial round of 256 x 256 tiles runs as quarter tiles: when
// the tile count leaves a last round of at most half the compute units
// (the 72B-class gate/up product: 1,848 tiles = 7 rounds + 56), those
// tiles are launched separately as 4 x as many 128 x 128 tiles on
// otherwise idle units.  Those finish in about half (not a quarter) of a
// full tile's time: a quarter tile's step has a quarter of the matrix work
// but the same load latency to hide, hence its deeper ring (8 stages of
// 16 KB).  Measured on the 72B-class gate/up product: the tail round
// 213 -> about 95 us.  Every output sums the same MFMAs in the same K
// order, so the results are the same bit for bit.  The same instantiation
// runs whole grids of up to 128 rows (launch_wide_epi).
struct WideTailCfg {
    static constexpr int BM = 128, BN = 128, WGM = 4, WGN = 2, KCS = 1, STAGES = 8;
};
static_assert(2 * WideTailCfg::BM == WideCfg::BM && 2 * WideTailCfg::BN == WideCfg::BN,
              "quarter tiles");

// For batches whose 256 x 256 grid would fill at most half the compute
// units: 256 rows by 4 pair blocks (8 waves of 64 x 64, ping-pong), six
// stages of 24 KB.
struct WideHalfCfg {
    static constexpr int BM = 256, BN = 128, WGM = 4, WGN = 2, KCS = 1, STAGES = 6;
};
constexpr int WIDE_CUS = 256;   // MI355X compute units: one 256 x 256 tile each per round

int wide_supported(const GemmArgs& g)
{
    // bf16 only; the A region of one tile must stay under 2 GB of byte
    // offsets and the packed B region of one tile under 4 GB.
    return g.dt == DT_BF16 && (int64_t)WideCfg::BM * g.lda * 2 < ((int64_t)1 << 31) &&
           (int64_t)(WideCfg::BN / 32) * g.geom.nkc * 2 * PIECE_BYTES < ((int64_t)1 << 32);
}

hipError_t wide_prepare()
{
    using C = WideCfg;
    using P = WidePhasedCfg;
    using T = WideTailCfg;
    hipError_t e =
        wide_attrs<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_SWIGLU, false, true>();
    if (e == hipSuccess)
        e = wide_attrs<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_PLAIN, false, true>();
    if (e == hipSuccess)
        e = wide_attrs<T::BM, T::BN, T::WGM, T::WGN, T::KCS, T::STAGES, EPI_SWIGLU>();
    if (e == hipSuccess)
        e = wide_attrs<T::BM, T::BN, T::WGM, T::WGN, T::KCS, T::STAGES, EPI_PLAIN>();
    if (e == hipSuccess)
        e = wide_attrs<P::BM, P::BN, P::WGM, P::WGN, P::KCS, P::STAGES, EPI_SWIGLU, true>();
    using H = WideHalfCfg;
    if (e == hipSuccess)
        e = wide_attrs<H::BM, H::BN, H::WGM, H::WGN, H::KCS, H::STAGES, EPI_SWIGLU, false, true>();
    if (e == hipSuccess)
        e = wide_attrs<H::BM, H::BN, H::WGM, H::WGN, H::KCS, H::STAGES, EPI_PLAIN, false, true>();
    return e;
}

// Workgroups of the grid launch_wide_epi runs for this product: the 256 x
// 256 tiles, or as many narrower tiles when those would fill at most half
// the compute units (its tail split leaves the count above that unchanged
// for the dispatcher's purpose).
int64_t wide_grid_tiles(const GemmArgs& g)
{
    using C = WideCfg;
    using T = WideTailCfg;
    using H = WideHalfCfg;
    const int64_t G = wide_full_grid<C::BM, C::BN, C::BN / 32>(g).blocks;
    if (G > WIDE_CUS / 2)
        return G;
    return g.M <= T::BM ? wide_full_grid<T::BM, T::BN, T::BN / 32>(g).blocks
                        : wide_full_grid<H::BM, H::BN, H::BN / 32>(g).blocks;
}

template <int EPI>
static hipError_t launch_wide_epi(const GemmArgs& g, hipStream_t s)
{
    using C = WideCfg;
    using T = WideTailCfg;
    WideGrid full = wide_full_grid<C::BM, C::BN, C::BN / 32>(g);
    const int G = full.blocks;
    // A grid of 256 x 256 tiles that fills at most half the compute units
    // (a batch of a few hundred rows: 112 tiles for the 8B-class gate/up
    // product up to 256 rows) leaves most of them idle while the product is
    // bound by the weight stream; the whole grid then runs as twice as many
    // narrower tiles: 128 x 128 up to 128 rows, 256 x 128 above.  Measured
    // on that shape: 65, 96, 128 rows 85.6, 87.9, 89.9 -> 57-61, 60-67,
    // 63-69 us; 192, 256 rows 95.7, 100.8 -> 88.4, 92.6 us.  Every output
    // sums the same MFMAs in the same K order, so the results are the same.
    if (G <= WIDE_CUS / 2) {
        if (g.M <= T::BM) {
            WideGrid q = wide_full_grid<T::BM, T::BN, T::BN / 32>(g);
            return launch_wide_cfg<T::BM, T::BN, T::WGM, T::WGN, T::KCS, T::STAGES, EPI>(
                g, s, C::GROUP_M, true, &q);
        }
        using H = WideHalfCfg;
        WideGrid q = wide_full_grid<H::BM, H::BN, H::BN / 32>(g);
        return launch_wide_cfg<H::BM, H::BN, H::WGM, H::WGN, H::KCS, H::STAGES, EPI, false, true>(
            g, s, C::GROUP_M, true, &q);
    }
    const int tail = G > WIDE_CUS ? G % WIDE_CUS : 0;
    if (tail == 0 || tail > WIDE_CUS / 2)
        return launch_wide_cfg<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI, false, true>(
            g, s, C::GROUP_M, true, &full);
    WideGrid head = full, rest = full;
    head.blocks = G - tail;
    rest.blocks = 4 * tail;
    rest.tail_base = G - tail;
    hipError_t e =
        launch_wide_cfg<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI, false, true>(
            g, s, C::GROUP_M, true, &head);
    if (e == hipSuccess)
        e = launch_wide_cfg<T::BM, T::BN, T::WGM, T::WGN, T::KCS, T::STAGES, EPI>(
            g, s, C::GROUP_M, true, &rest);
    return e;
}

hipError_t launch_wide(const GemmArgs& g, hipStream_t s)
{
    return g.epi == EPI_SWIGLU ? launch_wide_epi<EPI_SWIGLU>(g, s) : launch_wide_epi<EPI_PLAIN>(g, s);
}

hipError_t launch_wide_phased(const GemmArgs& g, hipStream_t s)
{
    using C = WidePhasedCfg;
    if (g.epi != EPI_SWIGLU)
        return hipErrorInvalidValue;
    return launch_wide_cfg<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_SWIGLU, true>(
        g, s, C::GROUP_M);
}

}  // namespace swg
