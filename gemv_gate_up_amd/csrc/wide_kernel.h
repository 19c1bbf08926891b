// wide_kernel.h -- the many-rows (prefill) MFMA GEMM, templated on its tile
// shape and pipeline depth; wide.hip instantiates the configuration used.
//
// This is the interleaved single-GEMM design of "Tile-Level Activation
// Overlap for Efficient LLM Inference" (Kernel-2): one GEMM over M x 2N x K
// on the fused weight, whose accumulator tile holds gate and up columns side
// by side; the epilogue stores silu(gate) * up, so the gate and up
// intermediates never reach HBM.  Built for gfx950 as follows:
//   * block tile BM x BN (BN counts fused columns: BN/32 pair blocks of 16
//     gate + 16 up columns); a pipeline stage holds KCS chunks of 32 K;
//   * both operands go global -> LDS with buffer_load ... lds (no VGPR
//     staging) into pieces that are exactly MFMA operand fragments, so every
//     ds_read_b128 is conflict free;
//   * STAGES LDS buffers in a ring, up to STAGES - 1 stages in flight; one
//     barrier per stage publishes stage t+1, whose fragments are then read
//     into registers behind stage t's MFMAs (v_mfma_f32_16x16x32_bf16), so
//     LDS latency hides behind matrix work;
//   * or (PP) the ping-pong schedule: the two waves of each SIMD alternate
//     between a phase of a whole step's MFMAs and a phase of fragment reads
//     and loads, one barrier per phase, so the matrix unit of every SIMD
//     always has one wave feeding it;
//   * pairing block = MFMA N fragment (16 columns): lane l holds gate and up
//     of the same output element, so the epilogue needs no lane exchange;
//   * tiles are remapped so each XCD (own L2) works through a compact group
//     of tiles that share A row panels and B column panels;
//   * the epilogue finishes every wave's values in registers at once, then
//     stages the tile through the freed ring and stores whole rows in
//     16-byte vectors;
//   * a launch may cover only part of the tile grid: the full rounds, or
//     (tail_base >= 0) the last partial round as quarter tiles.
// The down projection runs through the same kernel with a plain epilogue;
// with a residual (the MLP block) that epilogue stages fp32 products and adds
// the bias and the residual as the rows are written.
//
// PA: the left operand is in the packed activation layout of geometry.h, so
// that each of its loads is one contiguous 1 KB piece (a row-major tile
// reads a 64-byte fragment of each of 16 rows per load); measured about 7%
// faster on the 8B- and 72B-class prefill shapes.  PO: the tile's result
// is written in that layout (the h of the MLP, read back by the down
// product with PA).
//
// PHASED selects the other schedule of that paper (Kernel-1): the tile's
// accumulators hold gate columns only; the K loop runs once over the gate
// halves of the tile's pair blocks, silu is applied to the finished gate
// tile in registers while the first up stages are already in flight, and a
// second K loop over the up halves (re-reading A) ends in the product.  BN
// then counts output columns, and the result is bit-identical to the
// interleaved schedule: every accumulator sums the same MFMAs in the same
// K order.
#pragma once
#include <string.h>

#include "device_common.h"
#include "launch.h"

namespace swg {

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads (which would
// wait for every outstanding load, including the stages still in flight).
// LDS is written only by the buffer loads, whose completion each wave awaits
// with wait_vmcnt before arriving.  lgkmcnt(0) retires this wave's LDS reads
// before any wave may overwrite the buffer they read; it is issued through
// the builtin so that the compiler knows those reads are complete and does
// not wait again before MFMAs that use them.  The "memory" clobber keeps
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited
    asm volatile("s_barrier" ::: "memory");
}

constexpr uint32_t OOB_OFFSET = 0x80000000u;   // any offset >= num_records reads zero

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

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane, bypassing VGPRs;
// the address is base + voffset (per lane) + soffset (per wave, the K step).
// Issued through inline asm so that the compiler does not add a blanket
// vmcnt(0) before LDS reads; completion is awaited with wait_vmcnt.  The LDS
// base goes in through M0 as an operand, so the compiler writes M0 itself
// and knows its value.  A lane whose voffset alone is past num_records reads
// zero whatever soffset is.
__device__ __forceinline__ void load_lds16(const i32x4& srd, uint32_t voffset, uint32_t soffset,
                                           uint32_t lds_base) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(srd), "s"(soffset), "{m0}"(lds_base)
                 : "memory");
}

template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, bool PHASED = false>
struct WideShape {
    static constexpr int NW = WGM * WGN;
    static constexpr int THREADS = NW * 64;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int HALVES = PHASED ? 1 : 2;         // B halves loaded per stage
    static constexpr int PB_TILE = BN / (16 * HALVES);
    static constexpr int A_PIECES = (BM / 16) * KCS;      // [row block][chunk]
    static constexpr int B_PIECES = PB_TILE * KCS * HALVES;   // [pair block][chunk][half]
    static constexpr int PIECES = A_PIECES + B_PIECES;
    static constexpr int PPW = PIECES / NW;               // loads per wave per stage
    static constexpr int APW = A_PIECES / NW;
    static constexpr int STAGE_BYTES = PIECES * PIECE_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static_assert(PIECES % NW == 0 && A_PIECES % NW == 0, "pieces must split evenly");
    static_assert(PHASED || FN % 2 == 0, "a wave tile holds whole pair blocks");
    static_assert(STAGES >= 3, "stage t+1 must be in flight before step t starts");
    static_assert((STAGES - 2) * PPW < 64, "vmcnt budget");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int PPW, int MAXA>
__device__ __forceinline__ void wait_stage(int ahead) {
    // wait until at most min(ahead, MAXA) later stages of this wave remain
    // in flight
    if constexpr (MAXA > 0) {
        if (ahead >= MAXA) {
            wait_vmcnt<MAXA * PPW>();
            return;
        }
        wait_stage<PPW, MAXA - 1>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}

template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, int EPI, bool KTAIL, bool PHASED,
          bool PA, bool PO, bool PP = false>
__global__ void __launch_bounds__(WGM * WGN * 64, 1)
wide_bf16_kernel(const uint16_t* __restrict__ a, int64_t lda, int64_t kvalid, int M,
                 const uint16_t* __restrict__ w, int64_t nkc, int64_t npb,
                 uint16_t* __restrict__ out, int64_t ldo, int64_t ncols_out, int64_t out_nkc,
                 int tiles_m, int tiles_n, int group_m, int tail_base,
                 const uint16_t* __restrict__ resid, int64_t ldr, const uint16_t* __restrict__ bias)
{
    using S = WideShape<BM, BN, WGM, WGN, KCS, STAGES, PHASED>;
    constexpr int FM = S::FM, FN = S::FN, PPW = S::PPW, APW = S::APW, NW = S::NW;
    constexpr int A_PIECES = S::A_PIECES;
    static_assert(!PHASED || EPI == EPI_SWIGLU, "the phased schedule is for the gate/up pair");
    static_assert(!(PA && KTAIL), "packed activations are zero-padded along K");
    static_assert(!PO || EPI == EPI_SWIGLU, "packed output is the h of the gate/up pair");
    static_assert(!PP || (!PHASED && NW == 8), "ping-pong: one pass, two groups of four waves");

    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- tile coordinates: XCD-contiguous ranges, then grouped raster over
    // a grid of tiles_m x tiles_n tiles.  A tail launch (tail_base >= 0)
    // covers that grid's tiles from tail_base on, each as four quarter tiles
    // of this kernel's BM x BN (the grid's tiles are 2 BM x 2 BN).
    const bool tail = tail_base >= 0;
    int pid = tail ? tail_base + (int)(blockIdx.x >> 2) : (int)blockIdx.x;
    const int G = tiles_m * tiles_n;
    const int per_xcd = G / 8;
    if (pid < per_xcd * 8)
        pid = (pid % 8) * per_xcd + pid / 8;
    const int in_group = group_m * tiles_n;
    const int first_m = (pid / in_group) * group_m;
    const int gsz = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int tm = first_m + (pid % in_group) % gsz;
    const int tn = (pid % in_group) / gsz;

    const int sub = tail ? (int)(blockIdx.x & 3) : 0;
    const int m0 = tail ? tm * 2 * BM + (sub >> 1) * BM : tm * BM;
    const int64_t pb0 = (tail ? (int64_t)tn * 2 + (sub & 1) : (int64_t)tn) * S::PB_TILE;
    if (m0 >= M || pb0 >= npb)   // a quarter tile past the output (whole workgroup)
        return;
    const int rows_here = M - m0 < BM ? M - m0 : BM;
    // packed: the tile's row blocks, [row block][chunk] pieces of 1 KB
    const i32x4 ra =
        PA ? make_srd(a + (int64_t)(m0 / 16) * nkc * 512,
                      (uint32_t)(ceil_div(rows_here, 16) * nkc * PIECE_BYTES))
           : make_srd(a + (int64_t)m0 * lda, (uint32_t)((int64_t)rows_here * lda * 2));
    // pair blocks past the packed buffer read as zero
    const int64_t pbs_here = npb - pb0 < S::PB_TILE ? npb - pb0 : S::PB_TILE;
    const i32x4 rw = make_srd(w + pb0 * nkc * 2 * 512,
                              (uint32_t)(pbs_here * nkc * 2 * PIECE_BYTES));
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void_t*)smem;

    // ---- per-lane byte offsets of this wave's pieces in stage 0
    uint32_t off[PPW];
    int akk[APW > 0 ? APW : 1];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int q = wave + j * NW;
        if (j < APW) {
            const int rb = q / KCS, kc = q % KCS;
            const int row = rb * 16 + (lane & 15);
            const int kk = kc * 32 + (lane >> 4) * 8;
            akk[j] = kk;
            off[j] = PA ? (uint32_t)(((int64_t)rb * nkc + kc) * PIECE_BYTES + lane * 16)
                        : (uint32_t)(((int64_t)row * lda + kk) * 2);
        } else {
            const int qb = q - A_PIECES;
            const int pbl = qb / (KCS * S::HALVES), kc = (qb / S::HALVES) % KCS;
            const int half = PHASED ? 0 : qb & 1;
            off[j] = (uint32_t)(((int64_t)(pbl * nkc + kc) * 2 + half) * PIECE_BYTES + lane * 16);
        }
    }

    // K steps of one pass; the phased schedule makes two passes, the
    // second over the up halves.
    const int kpass = (int)(nkc / KCS);
    const int nsteps = PHASED ? 2 * kpass : kpass;

    // Issues piece j (of this wave's PPW pieces) of stage t into its ring
    // slot.  The K step advances through the scalar offset; only when K is
    // not a multiple of the stage depth (KTAIL) do A lanes past K take an
    // out-of-range offset so that they read zero.
    auto load_piece = [&](int t, int j) {
        const uint32_t base = smem_base + (uint32_t)(((unsigned)t % STAGES) * S::STAGE_BYTES);
        const int q = wave + j * NW;
        const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + q * PIECE_BYTES));
        const bool up_pass = PHASED && t >= kpass;
        const int tk = up_pass ? t - kpass : t;
        if (j < APW) {
            const uint32_t so = (uint32_t)(tk * (PA ? KCS * PIECE_BYTES : KCS * 64));
            uint32_t o = off[j];
            if (KTAIL && (int64_t)tk * (KCS * 32) + akk[j] >= kvalid)
                o = OOB_OFFSET;
            load_lds16(ra, o, so, dst);
        } else {
            const uint32_t so = (uint32_t)(tk * (KCS * 2 * PIECE_BYTES)) + (up_pass ? PIECE_BYTES : 0);
            load_lds16(rw, off[j], so, dst);
        }
    };
    auto load_stage = [&](int t) {
#pragma unroll
        for (int j = 0; j < PPW; ++j)
            load_piece(t, j);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    static_assert(KCS == 1, "one chunk per stage keeps the step count of a pass even");

    // Operand fragments in registers.  A fragments are double buffered;
    // each B fragment is refilled from the next stage as soon as the MFMAs
    // of the current stage that use it have been issued (B outer, A inner),
    // which keeps one B set live instead of two.
    struct AFrags {
        bf16x8 v[KCS][FM];
    };
    struct BFrags {
        bf16x8 v[KCS][FN];
    };
    auto stage_ptr = [&](int t) {
        return smem + ((unsigned)t % STAGES) * S::STAGE_BYTES + lane * 16;
    };
    auto read_a = [&](int t, AFrags& f) {
        const uint8_t* base = stage_ptr(t);
#pragma unroll
        for (int kc = 0; kc < KCS; ++kc)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                f.v[kc][fm] = *(const bf16x8*)(base + ((wm * FM + fm) * KCS + kc) * PIECE_BYTES);
    };
    auto read_b = [&](const uint8_t* base, int kc, int fn) {
        const int idx = wn * FN + fn;
        const int piece = PHASED ? A_PIECES + idx * KCS + kc
                                 : A_PIECES + ((idx >> 1) * KCS + kc) * 2 + (idx & 1);
        return *(const bf16x8*)(base + piece * PIECE_BYTES);
    };
    // MFMAs of one stage; with `refill`, stage t+1's fragments are read
    // behind them (its buffer was published by the preceding barrier).  The
    // loads of stage t+STAGES-1 are spread over the step, one piece after
    // each group of MFMAs: the inline asm that issues them bounds the
    // compiler's scheduling regions, so they stay interleaved with matrix
    // work instead of arriving in one burst (their ring slot was last read
    // two steps earlier).
    auto step = [&](int t, const AFrags& acur, AFrags& anext, BFrags& b, bool refill) {
        const uint8_t* nbase = stage_ptr(t + 1);
        const bool load = t + STAGES - 1 < nsteps;
        if (refill)
            read_a(t + 1, anext);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int kc = 0; kc < KCS; ++kc)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        acur.v[kc][fm], b.v[kc][fn], acc[fm][fn], 0, 0, 0);
            if (refill) {
#pragma unroll
                for (int kc = 0; kc < KCS; ++kc)
                    b.v[kc][fn] = read_b(nbase, kc, fn);
            }
            if (load) {
#pragma unroll
                for (int j = fn * PPW / FN; j < (fn + 1) * PPW / FN; ++j)
                    load_piece(t + STAGES - 1, j);
            }
        }
    };
    // Publishes stage t+1: its loads are done in every wave.
    auto advance = [&](int t) {
        const int rem = nsteps - 2 - t;
        wait_stage<PPW, STAGES - 2>((int)(rem < STAGES - 3 ? rem : STAGES - 3));
        barrier_lds();
    };

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nsteps)
            load_stage(s);
    {
        const int rem = nsteps - 1;
        wait_stage<PPW, STAGES - 2>((int)(rem < STAGES - 2 ? rem : STAGES - 2));
    }
    barrier_lds();
    f32x4 gs[PHASED ? FM : 1][PHASED ? FN : 1];   // silu(gate) of the phased schedule
    if constexpr (PP) {
        // Ping-pong: waves w and w + 4 share a SIMD; group 0 (waves 0-3)
        // and group 1 (waves 4-7) alternate phases, so on every SIMD one
        // wave issues a whole step of MFMAs back to back while the other
        // reads its next step's fragments from LDS and issues its share of
        // a stage's global -> LDS loads.  Each wave runs mem(0),
        // compute(0), mem(1), compute(1), ...; group 1 starts one phase
        // later.  A workgroup barrier ends every phase; before the barrier
        // that precedes a read of stage t by group 0 (the end of an odd
        // phase), every wave has its own loads of stage t complete, and
        // every barrier retires the wave's LDS reads, so the slot that a
        // mem phase reloads (stage t - 1's, last read in the phase before)
        // is free once the barrier between them has passed.  One fragment
        // set per wave: a mem phase refills the registers of the compute
        // phase before it.
        const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
        AFrags af;
        BFrags bf;
        auto mem = [&](int t) {
            read_a(t, af);
            const uint8_t* base = stage_ptr(t);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf.v[0][fn] = read_b(base, 0, fn);
            if (t + STAGES - 1 < nsteps)
                load_stage(t + STAGES - 1);
        };
        auto compute = [&]() {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af.v[0][fm], bf.v[0][fn],
                                                                          acc[fm][fn], 0, 0, 0);
        };
        // stage t + 1 complete in this wave (loads issued up to stage t + STAGES - 1)
        auto wait_next = [&](int t) {
            const int ahead = nsteps - 2 - t;
            wait_stage<PPW, STAGES - 2>(ahead < STAGES - 2 ? ahead : STAGES - 2);
        };
        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            barrier_lds();
            __builtin_amdgcn_sched_barrier(0);
        };
        if (grp)
            phase_end();
        for (int t = 0; t < nsteps; ++t) {
            mem(t);
            if (grp)
                wait_next(t);
            phase_end();
            compute();
            if (!grp)
                wait_next(t);
            phase_end();
        }
        if (!grp)
            phase_end();
    } else {
        AFrags a0, a1;
        BFrags b;
        read_a(0, a0);
        {
            const uint8_t* base0 = stage_ptr(0);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int kc = 0; kc < KCS; ++kc)
                    b.v[kc][fn] = read_b(base0, kc, fn);
        }
        // Two steps per trip so that both A sets stay in registers.  A pass
        // always has an even step count (K is padded to two chunks), so there
        // is no tail: the last refill reads a stale but in-bounds ring slot
        // whose values are never used.  No LDS read is conditional, so the
        // compiler's wait counts stay exact, and no peeled copy of the step
        // raises register pressure past the loop.
        for (int t = 0; t < kpass; t += 2) {
            advance(t);
            step(t, a0, a1, b, true);
            advance(t + 1);
            step(t + 1, a1, a0, b, true);
        }
        // Phased: the gate tile is finished; keep silu(gate) and run the up pass
        // (its first stages were issued during the gate pass).
        if constexpr (PHASED) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        gs[i][j][e] = silu(acc[i][j][e]);
                    acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            for (int t = kpass; t < nsteps; t += 2) {
                advance(t);
                step(t, a0, a1, b, true);
                advance(t + 1);
                step(t + 1, a1, a0, b, true);
            }
        }
    }

    // ---- epilogue: lane l holds rows 4*(l/16)+i of column l%16 of each
    // fragment.  Every wave first turns its accumulators into the finished
    // bf16 values in registers (silu(gate) * up, or the plain product plus
    // bias), all waves at once; the values are then staged in LDS (the ring
    // is free by now) as many wave-rows at a time as fit (the whole tile for
    // the gate/up product) and written to memory as whole rows of 16-byte
    // vectors, so every global write covers full lines.  A plain product
    // with a residual stages fp32 values instead (below).
    constexpr int OW = EPI == EPI_SWIGLU && !PHASED ? BN / 2 : BN;   // output columns of the tile
    constexpr int WOW = OW / WGN;                          // of one wave
    constexpr int FO = WOW / 16;                           // output fragments across a wave
    constexpr int LROW = OW + 8;                           // padded LDS row, elements
    constexpr int VPR = OW / 8;                            // 16-byte vectors per row
    constexpr int WR_FIT = S::LDS_BYTES / (S::WTM * LROW * 2);
    constexpr int WRP = WR_FIT >= WGM ? WGM : (WR_FIT >= WGM / 2 ? WGM / 2 : 1);   // wave-rows per pass
    constexpr int PROWS = WRP * S::WTM;                    // tile rows per pass
    static_assert(WRP >= 1 && WGM % WRP == 0 && PROWS * LROW * 2 <= S::LDS_BYTES,
                  "epilogue staging fits the ring");
    uint16_t* ep = (uint16_t*)smem;
    const int64_t col0 = EPI == EPI_SWIGLU ? pb0 * 16 : pb0 * 32;
    (void)gs;
    const int c = lane & 15;
    // fragment j of the wave holds output column wn * WOW + 16 * j + c
    // Plain products: the lane's bias values are loaded once, before any
    // is added.  Inside the output the arithmetic is the plain tail's
    // (bias, then residual, in fp32, one rounding); values outside it are
    // never stored.
    float bv[EPI == EPI_PLAIN ? FO : 1];
    if constexpr (EPI == EPI_PLAIN) {
#pragma unroll
        for (int j = 0; j < FO; ++j) {
            const int64_t gcol = col0 + wn * WOW + 16 * j + c;
            bv[j] = bias && gcol < ncols_out ? bf16_to_f32(bias[gcol]) : 0.f;
        }
    }
    (void)bv;
    if constexpr (EPI == EPI_PLAIN) {
        if (resid) {
            // With a residual (the MLP block's down product) the products
            // are staged in LDS as fp32, and the bias and the residual are
            // read like the output: whole 16-byte vectors, all of a thread's
            // vectors of a pass issued before the first is used.
            constexpr int LROWF = OW + 4;   // padded LDS row, floats
            constexpr int WRF_FIT = S::LDS_BYTES / (S::WTM * LROWF * 4);
            constexpr int WRPF = WRF_FIT >= WGM ? WGM : (WRF_FIT >= WGM / 2 ? WGM / 2 : 1);
            constexpr int PROWSF = WRPF * S::WTM;
            constexpr int ITER = PROWSF * VPR / S::THREADS;   // vectors per thread and pass
            static_assert(WRPF >= 1 && WGM % WRPF == 0 && PROWSF * LROWF * 4 <= S::LDS_BYTES,
                          "fp32 staging fits the ring");
            static_assert(ITER >= 1 && ITER * S::THREADS == PROWSF * VPR, "whole vectors per thread");
            float* epf = (float*)smem;
            // the tile's residual rows; a row past the output reads zeros
            // (at most 256 rows of 2^20 columns: well inside 32-bit offsets)
            const uint32_t rbytes = (uint32_t)((int64_t)rows_here * ldr * 2);
            const __amdgpu_buffer_rsrc_t rres = make_rsrc(resid + (int64_t)m0 * ldr, rbytes);
            // a thread's columns are the same in every pass and vector
            static_assert(S::THREADS % VPR == 0, "fixed columns per thread");
            float bcol[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t col = col0 + (threadIdx.x % VPR) * 8 + e;
                bcol[e] = bias && col < ncols_out ? bf16_to_f32(bias[col]) : 0.f;
            }
#pragma unroll 1
            for (int pass = 0; pass < WGM / WRPF; ++pass) {
                i32x4 rr[ITER];
#pragma unroll
                for (int it = 0; it < ITER; ++it) {
                    const int v = threadIdx.x + it * S::THREADS;
                    const int r = pass * PROWSF + v / VPR;
                    const uint32_t off =
                        r < rows_here ? (uint32_t)(((int64_t)r * ldr + col0 + (v % VPR) * 8) * 2)
                                      : rbytes;
                    rr[it] = __builtin_amdgcn_raw_buffer_load_b128(rres, off, 0, 0);
                }
                __syncthreads();   // ring reads (first pass) or previous reads (later) are done
                if (wm / WRPF == pass) {
                    const int rbase = (wm % WRPF) * S::WTM;
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int j = 0; j < FO; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = rbase + fm * 16 + (lane >> 4) * 4 + i;
                                epf[r * LROWF + wn * WOW + 16 * j + c] = acc[fm][j][i];
                            }
                }
                __syncthreads();
#pragma unroll
                for (int it = 0; it < ITER; ++it) {
                    const int v = threadIdx.x + it * S::THREADS;
                    const int r = v / VPR, cv = v % VPR;
                    const int row = m0 + pass * PROWSF + r;
                    const int64_t col = col0 + cv * 8;
                    if (row < M && col < ncols_out) {
                        const float* src = epf + r * LROWF + cv * 8;
                        const i32x4 rv = rr[it];
                        i32x4 o;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t w = (uint32_t)rv[q];
                            float lo = src[2 * q], hi = src[2 * q + 1];
                            if (bias) {
                                lo += bcol[2 * q];
                                hi += bcol[2 * q + 1];
                            }
                            lo += bf16_to_f32((uint16_t)w);
                            hi += bf16_to_f32((uint16_t)(w >> 16));
                            o[q] = (int)((uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16));
                        }
                        *(i32x4*)(out + (int64_t)row * ldo + col) = o;
                    }
                }
            }
            return;
        }
    }
    uint16_t res[FM][FO][4];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int j = 0; j < FO; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v;
                if constexpr (PHASED) {
                    v = gs[fm][j][i] * acc[fm][j][i];
                } else if constexpr (EPI == EPI_SWIGLU) {
                    v = silu(acc[fm][2 * j][i]) * acc[fm][2 * j + 1][i];
                } else {
                    v = acc[fm][j][i];
                    if (bias)
                        v += bv[j];
                }
                res[fm][j][i] = f32_to_bf16(v);
            }
#pragma unroll 1
    for (int pass = 0; pass < WGM / WRP; ++pass) {
        __syncthreads();   // ring reads (first pass) or previous stores (later) are done
        if (wm / WRP == pass) {
            const int rbase = (wm % WRP) * S::WTM;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int j = 0; j < FO; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = rbase + fm * 16 + (lane >> 4) * 4 + i;
                        ep[r * LROW + wn * WOW + 16 * j + c] = res[fm][j][i];
                    }
        }
        __syncthreads();
        if constexpr (PO) {
            // one 1 KB piece per 64 consecutive threads: rows padded to 16
            // (the padded rows hold the zero products of zero rows) and
            // chunks up to out_nkc
            constexpr int CPR = OW / 32;   // chunks across the tile
            static_assert(PROWS % 16 == 0 && OW % 32 == 0, "whole pieces per pass");
            const int64_t rows_pad = round_up(M, 16);
            for (int v = threadIdx.x; v < PROWS * VPR; v += S::THREADS) {
                const int l = v & 63, p = v >> 6;
                const int r = (p / CPR) * 16 + (l & 15), ch = p % CPR, kg = l >> 4;
                const int64_t row = m0 + pass * PROWS + r;
                const int64_t col = col0 + ch * 32 + kg * 8;
                if (row < rows_pad && col < out_nkc * 32)
                    *(i32x4*)(out + act_packed_index(row, col, out_nkc)) =
                        *(const i32x4*)(ep + r * LROW + ch * 32 + kg * 8);
            }
        } else {
            for (int v = threadIdx.x; v < PROWS * VPR; v += S::THREADS) {
                const int r = v / VPR, cv = v % VPR;
                const int row = m0 + pass * PROWS + r;
                const int64_t col = col0 + cv * 8;
                if (row < M && col < ncols_out)
                    *(i32x4*)(out + (int64_t)row * ldo + col) =
                        *(const i32x4*)(ep + r * LROW + cv * 8);
            }
        }
    }
}

// Raises one instantiation's dynamic LDS limit to its ring size, once per
// process (a function-local static: thread-safe, and the host call is made
// outside any later stream capture when the library's prepare step runs
// first).
template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, int EPI, bool KTAIL, bool PHASED,
          bool PA, bool PO, bool PP = false>
static hipError_t wide_attr()
{
    using S = WideShape<BM, BN, WGM, WGN, KCS, STAGES, PHASED>;
    static const hipError_t e = hipFuncSetAttribute(
        (const void*)&wide_bf16_kernel<BM, BN, WGM, WGN, KCS, STAGES, EPI, KTAIL, PHASED, PA, PO, PP>,
        hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
    return e;
}

// Which tiles one launch covers: the first `blocks` tiles of a tiles_m x
// tiles_n grid of BM x BN tiles, or (tail_base >= 0) the tiles from
// tail_base on of a grid of 2 BM x 2 BN tiles, as 4 * blocks quarter tiles.
struct WideGrid {
    int tiles_m, tiles_n, blocks, tail_base;
};

template <int BM, int BN, int PB_TILE>
WideGrid wide_full_grid(const GemmArgs& g)
{
    WideGrid r;
    r.tiles_m = (int)ceil_div(g.M, BM);
    r.tiles_n = (int)ceil_div(ceil_div(g.ncols_out, g.geom.cols_per_pb), PB_TILE);
    r.blocks = r.tiles_m * r.tiles_n;
    r.tail_base = -1;
    return r;
}

// Host launcher for one instantiation.
template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, int EPI, bool KTAIL, bool PHASED,
          bool PA, bool PO, bool PP = false>
static hipError_t launch_wide_inst(const GemmArgs& g, hipStream_t s, int group_m, bool launch,
                                   const WideGrid* grid)
{
    using S = WideShape<BM, BN, WGM, WGN, KCS, STAGES, PHASED>;
    const hipError_t e = wide_attr<BM, BN, WGM, WGN, KCS, STAGES, EPI, KTAIL, PHASED, PA, PO, PP>();
    if (e != hipSuccess || !launch)
        return e;
    const WideGrid gr = grid ? *grid : wide_full_grid<BM, BN, S::PB_TILE>(g);
    if (gr.blocks <= 0)
        return hipSuccess;
    wide_bf16_kernel<BM, BN, WGM, WGN, KCS, STAGES, EPI, KTAIL, PHASED, PA, PO, PP>
        <<<dim3((unsigned)gr.blocks), dim3(S::THREADS), S::LDS_BYTES, s>>>(
            (const uint16_t*)g.a, g.lda, g.geom.K, (int)g.M, (const uint16_t*)g.w, g.geom.nkc,
            g.geom.npb, (uint16_t*)g.out, g.ldo, g.ncols_out, g.out_nkc, gr.tiles_m, gr.tiles_n,
            group_m, gr.tail_base, (const uint16_t*)g.resid, g.ldr, (const uint16_t*)g.bias);
    return hipGetLastError();
}

// Picks the instantiation for the operand layouts of g: packed or row-major
// activations, packed or row-major output.  Row-major activations take the
// K-tail variant whenever the weight's chunks reach past K (K not a whole
// number of stages, or K padded by a chunk to the weight's even chunk
// count): the lanes of those chunks would otherwise read the next row's
// first values, or past the end of the last row, and multiply them by the
// zero padding of the weights, where an Inf or NaN would still poison the
// sum.  With launch = false it only sets the launch attribute of that
// instantiation.
template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, int EPI, bool PHASED, bool PO,
          bool PP = false>
static hipError_t launch_wide_out(const GemmArgs& g, hipStream_t s, int group_m, bool launch,
                                  const WideGrid* grid)
{
    if (g.a_packed)
        return launch_wide_inst<BM, BN, WGM, WGN, KCS, STAGES, EPI, false, PHASED, true, PO, PP>(
            g, s, group_m, launch, grid);
    if (g.geom.K == g.geom.nkc * 32)
        return launch_wide_inst<BM, BN, WGM, WGN, KCS, STAGES, EPI, false, PHASED, false, PO, PP>(
            g, s, group_m, launch, grid);
    return launch_wide_inst<BM, BN, WGM, WGN, KCS, STAGES, EPI, true, PHASED, false, PO, PP>(
        g, s, group_m, launch, grid);
}

template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, int EPI, bool PHASED = false,
          bool PP = false>
hipError_t launch_wide_cfg(const GemmArgs& g, hipStream_t s, int group_m, bool launch = true,
                           const WideGrid* grid = nullptr)
{
    if constexpr (EPI == EPI_SWIGLU) {
        if (g.out_nkc > 0)
            return launch_wide_out<BM, BN, WGM, WGN, KCS, STAGES, EPI, PHASED, true, PP>(
                g, s, group_m, launch, grid);
    }
    return launch_wide_out<BM, BN, WGM, WGN, KCS, STAGES, EPI, PHASED, false, PP>(
        g, s, group_m, launch, grid);
}

// Sets the launch attribute of every instantiation of one configuration.
template <int BM, int BN, int WGM, int WGN, int KCS, int STAGES, int EPI, bool PHASED = false,
          bool PP = false>
hipError_t wide_attrs()
{
    GemmArgs g;
    memset(&g, 0, sizeof g);
    hipError_t e = hipSuccess;
    for (int variant = 0; variant < 6 && e == hipSuccess; ++variant) {
        g.a_packed = variant % 3 == 2;
        g.geom.K = variant % 3 == 1 ? 1 : 0;   // K tail or not
        g.out_nkc = variant / 3;
        e = launch_wide_cfg<BM, BN, WGM, WGN, KCS, STAGES, EPI, PHASED, PP>(g, nullptr, 0, false);
    }
    return e;
}

}  // namespace swg
