// wide.hip -- the many-rows (prefill) path: one bf16 MFMA GEMM over the
// fused weight with the SiLU-times-up epilogue applied in registers.
//
// This is the interleaved single-GEMM design of "Tile-Level Activation
// Overlap for Efficient LLM Inference" (Kernel-2): one GEMM over M x 2N x K
// on the fused weight, whose accumulator tile holds gate and up columns
// side by side; the epilogue stores silu(gate) * up, so the gate and up
// intermediates never reach HBM.  On gfx950 it is built as follows:
//   * block tile BM x BN (BN counts fused columns: BN/32 pair blocks of 16
//     gate + 16 up columns) with K steps of 64;
//   * both operands are copied global -> LDS with buffer_load ... lds (no
//     VGPR staging), into a layout where every 1 KB piece is exactly one
//     MFMA operand fragment, so each ds_read_b128 is conflict free;
//   * two LDS stages: the loads of step t+1 are in flight while step t runs
//     on v_mfma_f32_16x16x32_bf16;
//   * pairing block = MFMA N fragment (16 columns), so lane l holds gate and
//     up of the same output element and the epilogue needs no lane exchange;
//   * tiles are remapped so that each XCD (own L2) works on a compact group
//     of tiles sharing A row panels and B column panels.
// The down projection runs through the same kernel with a plain epilogue.
#include "device_common.h"
#include "launch.h"

namespace swg {

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

constexpr uint32_t OOB_OFFSET = 0x80000000u;   // any offset >= num_records reads zero

// Workgroup barrier without the release fence of __syncthreads (which
// would wait for every outstanding load, including the next stage's).
// LDS is only written by the buffer loads, whose completion each wave
// awaits with wait_vmcnt before arriving; the "memory" clobber keeps the
// compiler from moving LDS reads across it.
__device__ __forceinline__ void barrier_only() {
    asm volatile("s_barrier" ::: "memory");
}

// Raw buffer descriptor (base, stride 0, num_records bytes) in four SGPRs.
__device__ __forceinline__ i32x4 make_srd(const void* base, uint32_t num_bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
    r.z = __builtin_amdgcn_readfirstlane((int)num_bytes);
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane, bypassing VGPRs.
// Issued through inline asm so that the compiler does not add a blanket
// vmcnt(0) before every LDS read; completion is awaited explicitly with
// wait_vmcnt before the barrier that publishes a stage.
__device__ __forceinline__ void load_lds16(const i32x4& srd, uint32_t voffset, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(srd), "s"(lds_base)
                 : "memory", "m0");
}

template <int BM, int BN, int WGM, int WGN, int EPI>
__global__ void __launch_bounds__(WGM * WGN * 64, 1)
wide_bf16_kernel(const uint16_t* __restrict__ a, int64_t lda, int64_t kvalid, int M,
                 const uint16_t* __restrict__ w, int64_t nkc,
                 uint16_t* __restrict__ out, int64_t ldo, int64_t ncols_out,
                 int tiles_m, int tiles_n, int group_m)
{
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int PB_TILE = BN / 32;
    constexpr int A_PIECES = (BM / 16) * 2;       // [row block][chunk]
    constexpr int B_PIECES = PB_TILE * 4;         // [pair block][chunk][half]
    constexpr int PIECES = A_PIECES + B_PIECES;
    constexpr int PPW = PIECES / NW;              // pieces each wave loads per stage
    constexpr int APW = A_PIECES / NW;            // of which A pieces
    static_assert(PIECES % NW == 0 && A_PIECES % NW == 0, "piece split");
    static_assert(FN % 2 == 0, "wave tile must hold whole pair blocks");
    static_assert(PPW < 32, "vmcnt budget");

    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- tile coordinates: XCD-contiguous ranges, then grouped raster
    int pid = blockIdx.x;
    const int G = tiles_m * tiles_n;
    const int per_xcd = G / 8;
    if (pid < per_xcd * 8)
        pid = (pid % 8) * per_xcd + pid / 8;
    const int in_group = group_m * tiles_n;
    const int first_m = (pid / in_group) * group_m;
    const int gsz = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int tm = first_m + (pid % in_group) % gsz;
    const int tn = (pid % in_group) / gsz;

    const int m0 = tm * BM;
    const int64_t pb0 = (int64_t)tn * PB_TILE;
    const int rows_here = M - m0 < BM ? M - m0 : BM;
    const i32x4 ra = make_srd(a + (int64_t)m0 * lda, (uint32_t)((int64_t)rows_here * lda * 2));
    const i32x4 rw =
        make_srd(w + pb0 * nkc * 2 * 512, (uint32_t)((int64_t)PB_TILE * nkc * 2 * PIECE_BYTES));
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void_t*)smem;

    // ---- per-lane byte offsets of this wave's pieces at K step 0
    uint32_t off[PPW];
    int64_t akk[APW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int q = wave + j * NW;
        if (j < APW) {
            const int rb = q >> 1, kc = q & 1;
            const int row = rb * 16 + (lane & 15);
            const int kk = kc * 32 + (lane >> 4) * 8;
            akk[j] = kk;
            off[j] = (uint32_t)(((int64_t)row * lda + kk) * 2);
        } else {
            const int qb = q - A_PIECES;
            const int pbl = qb >> 2, kc = (qb >> 1) & 1, half = qb & 1;
            off[j] = (uint32_t)(((int64_t)(pbl * nkc + kc) * 2 + half) * PIECE_BYTES + lane * 16);
        }
    }

    auto load_stage = [&](int64_t t, int buf) {
        const uint32_t base = smem_base + (uint32_t)(buf * PIECES * PIECE_BYTES);
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
            const int q = wave + j * NW;
            const uint32_t dst =
                (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + q * PIECE_BYTES));
            if (j < APW) {
                const int64_t k = t * 64 + akk[j];
                const uint32_t o = k < kvalid ? off[j] + (uint32_t)(t * 128) : OOB_OFFSET;
                load_lds16(ra, o, dst);
            } else {
                load_lds16(rw, off[j] + (uint32_t)(t * 4 * PIECE_BYTES), dst);
            }
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nsteps = nkc / 2;
    load_stage(0, 0);
    for (int64_t t = 0; t < nsteps; ++t) {
        const int cur = (int)(t & 1);
        if (t + 1 < nsteps) {
            load_stage(t + 1, cur ^ 1);
            wait_vmcnt<PPW>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_only();
        const uint8_t* base = smem + cur * PIECES * PIECE_BYTES + lane * 16;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int rb = wm * FM + fm;
                af[fm] = *(const bf16x8*)(base + (rb * 2 + kc) * PIECE_BYTES);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int idx = wn * FN + fn;
                const int piece = A_PIECES + ((idx >> 1) * 2 + kc) * 2 + (idx & 1);
                bfr[fn] = *(const bf16x8*)(base + piece * PIECE_BYTES);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn],
                                                                          acc[fm][fn], 0, 0, 0);
        }
        barrier_only();
    }

    // ---- epilogue: lane l holds rows 4*(l/16)+i of column l%16 of each fragment
    const int c = lane & 15;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp) {
            const int64_t pb = pb0 + (wn * FN) / 2 + jp;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
                if (row >= M)
                    continue;
                uint16_t* orow = out + (int64_t)row * ldo;
                if (EPI == EPI_SWIGLU) {
                    const int64_t n = pb * 16 + c;
                    if (n < ncols_out)
                        orow[n] = f32_to_bf16(silu(acc[fm][2 * jp][i]) * acc[fm][2 * jp + 1][i]);
                } else {
                    const int64_t j = pb * 32 + c;
                    if (j < ncols_out)
                        orow[j] = f32_to_bf16(acc[fm][2 * jp][i]);
                    if (j + 16 < ncols_out)
                        orow[j + 16] = f32_to_bf16(acc[fm][2 * jp + 1][i]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch
struct WideCfg {
    static constexpr int BM = 256, BN = 256, WGM = 2, WGN = 2;
    static constexpr int PIECES = (BM / 16) * 2 + (BN / 32) * 4;
    static constexpr int LDS_BYTES = 2 * PIECES * PIECE_BYTES;
};

int wide_supported(const GemmArgs& g)
{
    // bf16 only; the packed weights must cover whole BN tiles and the A
    // region of one tile must stay under 2 GB of byte offsets.
    return g.dt == DT_BF16 && (g.geom.npb * 32) % WideCfg::BN == 0 &&
           (int64_t)WideCfg::BM * g.lda * 2 < ((int64_t)1 << 31) &&
           g.geom.npb * 32 <= ((int64_t)1 << 30);
}

template <int EPI>
static hipError_t go_wide(const GemmArgs& g, hipStream_t s)
{
    using C = WideCfg;
    static bool attr_set = false;   // benign race: every writer stores the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            (const void*)&wide_bf16_kernel<C::BM, C::BN, C::WGM, C::WGN, EPI>,
            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int tiles_m = (int)ceil_div(g.M, C::BM);
    const int tiles_n = (int)ceil_div(ceil_div(g.ncols_out, g.geom.cols_per_pb) * 32, C::BN);
    const int group_m = 8;
    wide_bf16_kernel<C::BM, C::BN, C::WGM, C::WGN, EPI>
        <<<dim3((unsigned)(tiles_m * tiles_n)), dim3(C::WGM * C::WGN * 64), C::LDS_BYTES, s>>>(
            (const uint16_t*)g.a, g.lda, g.geom.K, (int)g.M, (const uint16_t*)g.w, g.geom.nkc,
            (uint16_t*)g.out, g.ldo, g.ncols_out, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

hipError_t launch_wide(const GemmArgs& g, hipStream_t s)
{
    return g.epi == EPI_SWIGLU ? go_wide<EPI_SWIGLU>(g, s) : go_wide<EPI_PLAIN>(g, s);
}

}  // namespace swg
