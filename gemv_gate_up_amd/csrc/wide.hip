// wide.hip -- instantiates the many-rows MFMA GEMM of wide_kernel.h with the
// tile shape and pipeline depth measured best on MI355X.
#include "wide_kernel.h"

namespace swg {

// 256 x 256 fused-column tile, 8 waves (2 per SIMD) of 64 x 128, stages of
// one 32-K chunk, four stages in the LDS ring (up to three in flight).
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
    hipError_t e = wide_attrs<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_SWIGLU>();
    if (e == hipSuccess)
        e = wide_attrs<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_PLAIN>();
    if (e == hipSuccess)
        e = wide_attrs<P::BM, P::BN, P::WGM, P::WGN, P::KCS, P::STAGES, EPI_SWIGLU, true>();
    return e;
}

hipError_t launch_wide(const GemmArgs& g, hipStream_t s)
{
    using C = WideCfg;
    if (g.epi == EPI_SWIGLU)
        return launch_wide_cfg<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_SWIGLU>(
            g, s, C::GROUP_M);
    return launch_wide_cfg<C::BM, C::BN, C::WGM, C::WGN, C::KCS, C::STAGES, EPI_PLAIN>(
        g, s, C::GROUP_M);
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
