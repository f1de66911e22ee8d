// gemm_bf16_packed.hip -- mixed precision in two steps: a kernel that rounds
// an FP32 operand to bf16 once and stores it k-contiguous ("packing"), and a
// matrix-core product of two packed operands with FP32 sums and FP32 C.
//
// The Smallem page ("Rendre le GPU rapide", section "Les Tensor Cores")
// rounds only the operands of each product to 16 bits and keeps sums and
// tensors in FP32; its comparison with PyTorch notes that PyTorch keeps the
// 16-bit copies of its operands where Smallem converts on every read.  The
// fused path (gemm_bf16.hip) converts on every read; this file is the other
// choice.  Rounding once pays off on gfx950 because a bf16 stage is short:
// a 256 x 256 x 32 stage is about a thousand matrix-core cycles, too short
// for register-staged FP32 loads to hide their latency, while bf16 tiles
// copied straight into LDS (buffer loads into LDS on a scalar descriptor;
// GEMM_PACKED_BUFFER_DMA 0 builds the global_load_lds form) move half the
// bytes with no register or LDS-write instructions.
//
// Product kernel layout:
//  * A BM x BN tile of C per workgroup of WAVES_M x WAVES_N waves; each wave
//    owns FM x FN blocks of 32 x 32 in accumulator registers.  One
//    v_mfma_f32_32x32x16_bf16 covers 16 k (32768 flops per wave
//    instruction); lanes 0-31 supply k slots 0-7 and lanes 32-63 slots 8-15,
//    each as one 16-byte LDS read, for A and B alike.
//  * Both packed operands hold k along their rows, so an LDS stage is BM (or
//    BN) rows of BK bf16, unpadded, with 16-byte vectors XOR-swizzled within
//    each row (the DMA writes 1 KB contiguously; the swizzle replaces the
//    padding that section 3.6 of the course page "3 . La memoire partagee"
//    uses against bank conflicts).
//  * Interior tiles copy full stages by DMA, NBUF - 1 stages ahead (in
//    effect one: the barrier's release fence drains every copy), one
//    barrier per stage; edge tiles and a partial last stage go through
//    registers with every element predicated (zero outside the matrix).
//  * The 256 x 256 and 256 x 128 tiles keep one accumulator: each MFMA adds
//    16 exact products before it rounds, so the relative error of a K = 8192
//    product stays near 5e-7.  The 128 x 128 tile, also used past K = 16384,
//    sums runs of FOLD stages into a fresh partial first.
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kWave = 64;
constexpr int kBlk = 32;

template <int V>
struct Int {
    static constexpr int value = V;
};
template <bool V>
struct Bool {
    static constexpr bool value = V;
};

// Interior stages are copied with buffer loads (1) or global loads (0)
// into LDS.
#ifndef GEMM_PACKED_BUFFER_DMA
#define GEMM_PACKED_BUFFER_DMA 1
#endif
#ifndef GEMM_PACKED_DEEP
#define GEMM_PACKED_DEEP 1
#endif
#ifndef GEMM_PACKED_RUNTIME_BUFFER
#define GEMM_PACKED_RUNTIME_BUFFER 1
#endif

template <int N, int I = 0, class F>
__device__ __forceinline__ void unroll_for(F &&f)
{
    if constexpr (I < N) {
        f(Int<I>{});
        unroll_for<N, I + 1>(f);
    }
}

// BM x BN of C per workgroup, BK bf16 per stage, WAVES_M x WAVES_N waves,
// NBUF LDS stage buffers (copies issued NBUF - 1 stages ahead), GROUP_M tile-rows per
// group of the launch order, FOLD stages per accumulation chunk (0: one
// running accumulator), STAGGER: the second half of the waves issues its
// share of the next stage's copies after the first MFMA step instead of
// right after the barrier, so the two waves of a SIMD do not both stall on
// copy issue at once.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int NBUF_, int GROUP_M_, int FOLD_,
          int STAGGER_ = 0>
struct Config {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int waves_n = WAVES_N_;
    static constexpr int waves = WAVES_M_ * WAVES_N_;
    static constexpr int threads = kWave * waves;
    static constexpr int WM = BM / WAVES_M_, WN = BN / WAVES_N_;
    static constexpr int FM = WM / kBlk, FN = WN / kBlk;
    static constexpr int nbuf = NBUF_, group_m = GROUP_M_, fold = FOLD_;
    static constexpr bool stagger = STAGGER_;
    static_assert(WM % kBlk == 0 && WN % kBlk == 0, "wave tiles are whole MFMA blocks");
    static_assert(BK == 32 || BK == 64, "a stage row is 4 or 8 16-byte vectors");
    static_assert(NBUF_ >= 2 && NBUF_ <= 4, "2-4 stage buffers");
    static_assert(FOLD_ == 0 || NBUF_ % FOLD_ == 0 || FOLD_ % NBUF_ == 0,
                  "a chunk divides, or is a multiple of, the buffer cycle");
};

// One packed operand's LDS tile for one stage: P rows of BK bf16.  16-byte
// vector v of row r sits at vector slot r * vpr + (v ^ swz(r)).
template <class Cfg, int P>
struct Tile {
    static constexpr int vpr = Cfg::BK / 8;          // 16-byte vectors per row
    static constexpr int vecs = P * vpr;
    static constexpr int bytes = 16 * vecs;
    static constexpr int chunks = vecs / kWave;      // 1 KB DMA pieces
    static constexpr int dma_per_wave = chunks / Cfg::waves;
    static_assert(chunks % Cfg::waves == 0, "DMA pieces split evenly over the waves");
    static constexpr int per_thread = (vecs + Cfg::threads - 1) / Cfg::threads;
    static_assert(vecs % Cfg::threads == 0, "register staging splits evenly");

    // A fragment read takes vector 2g + h of 32 consecutive rows (h = lane
    // half).  With 4 vectors per row (64-byte rows) ((r >> 1) ^ (r >> 2)) & 3
    // puts any 8 consecutive rows, and any 16 consecutive rows taken four
    // apart in r & 3, in distinct 16-byte bank groups; with 8 vectors per
    // row (r & 7) ^ ((r >> 3) & 1) does the same.  So reads are free of bank
    // conflicts whether the LDS serves 8 or 16 lanes of a 16-byte read per
    // cycle.
    __device__ static __forceinline__ int swz(int r)
    {
        if (vpr == 4) return ((r >> 1) ^ (r >> 2)) & 3;
        return ((r & 7) ^ ((r >> 3) & 1)) & 7;
    }
    __device__ static __forceinline__ int slot(int r, int v) { return r * vpr + (v ^ swz(r)); }

    // Byte offset, from the stage's origin in the packed operand, of the
    // vector this lane copies in its wave's DMA piece q: lane l of piece c
    // fills vector slot 64c + l and fetches the vector the swizzle puts
    // there.  The caller guarantees P * ld * 2 < 2^32.
    __device__ static __forceinline__ uint32_t dma_offset(int64_t ld, int wave, int lane, int q)
    {
        const int s = (wave * dma_per_wave + q) * kWave + lane;
        const int r = s / vpr;
        const int v = (s % vpr) ^ swz(r);
        return uint32_t((int64_t(r) * ld + 8 * v) * 2);
    }
    __device__ static __forceinline__ void dma(char *lds, const char *origin,
                                               const uint32_t (&off)[dma_per_wave], int wave)
    {
        if (GEMM_LDS_POISON) {
#pragma unroll
            for (int q = 0; q < dma_per_wave; ++q)
                poison16(lds + 1024 * (wave * dma_per_wave + q) + 16 * (threadIdx.x % kWave));
            poison_wait();
        }
#pragma unroll
        for (int q = 0; q < dma_per_wave; ++q)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const float *>(origin + off[q]),
                                             reinterpret_cast<float *>(lds + 1024 * (wave * dma_per_wave + q)),
                                             16, 0, 0);
    }

    // The same copies as buffer loads: the stage's offset along k is an
    // SGPR offset (soff) on a raw buffer descriptor of the operand tile's
    // first row (no stride, no range limit: the host keeps every offset
    // below 2^32; the data format untyped loads need on this family), so
    // each lane keeps only its 32-bit offsets, where global loads would keep
    // a 64-bit address per copy live across the loop.
    __device__ static __forceinline__ void dma_buffer(char *lds, const char *row0, uint32_t soff,
                                                      const uint32_t (&off)[dma_per_wave], int wave)
    {
        if (GEMM_LDS_POISON) {
#pragma unroll
            for (int q = 0; q < dma_per_wave; ++q)
                poison16(lds + 1024 * (wave * dma_per_wave + q) + 16 * (threadIdx.x % kWave));
            poison_wait();
        }
        const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(row0), short(0),
                                                            int(0xFFFFFFFFu), int(0x00020000));
#pragma unroll
        for (int q = 0; q < dma_per_wave; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void *)(lds + 1024 * (wave * dma_per_wave + q)), 16, off[q],
                soff, 0, 0);
    }

    // Register staging: vector i = threadIdx.x + threads * q of the tile is
    // row i / vpr, k = 8 * (i % vpr) .. +7.  Elements outside rows x cols of
    // the packed operand (rows along m or n, cols along k) read as zero.
    // VEC: the operand allows aligned 16-byte loads.
    template <bool VEC>
    __device__ static __forceinline__ void load(const u16 *base, int64_t ld, int rows, int cols, int r0,
                                                int k0, v4u (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            const int i = int(threadIdx.x) + Cfg::threads * q;
            const int r = r0 + i / vpr, k = k0 + 8 * (i % vpr);
            const u16 *src = base + int64_t(r) * ld + k;
            if (VEC && r < rows && k + 7 < cols) {
                reg[q] = *reinterpret_cast<const v4u *>(src);
            } else {
                v4u x;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const unsigned lo = (r < rows && k + 2 * w < cols) ? src[2 * w] : 0u;
                    const unsigned hi = (r < rows && k + 2 * w + 1 < cols) ? src[2 * w + 1] : 0u;
                    x[w] = lo | (hi << 16);  // the lower address is the low half
                }
                reg[q] = x;
            }
        }
    }
    __device__ static __forceinline__ void store(char *lds, const v4u (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            const int i = int(threadIdx.x) + Cfg::threads * q;
            *reinterpret_cast<v4u *>(lds + 16 * slot(i / vpr, i % vpr)) = reg[q];
        }
    }
    // The race-detection build's NaN over the bytes store() will write.
    __device__ static __forceinline__ void poison(char *lds)
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            const int i = int(threadIdx.x) + Cfg::threads * q;
            poison16(lds + 16 * slot(i / vpr, i % vpr));
        }
    }

    // The 8 k values (16 g + 8 h .. +7) of row p for MFMA step g.
    __device__ static __forceinline__ v8bf fragment(const char *lds, int p, int g, int h)
    {
        return *reinterpret_cast<const v8bf *>(lds + 16 * slot(p, 2 * g + h));
    }

    // A lane reads rows p0 + 32 i (i = 0, 1, ...).  The swizzle depends only
    // on r mod 16, so rows 32 apart share it: one byte offset per step g
    // serves every i, and row p0 + 32 i lies a constant 32 * 16 * vpr bytes
    // further (an immediate offset of the LDS read), which keeps the
    // per-lane address registers at BK / 16.
    static constexpr int kSteps = Cfg::BK / 16;
    static constexpr int kRowBytes = 16 * vpr;
    struct Lane {
        uint32_t off[kSteps];
    };
    __device__ static __forceinline__ Lane lane_offsets(int p0, int h)
    {
        Lane f;
#pragma unroll
        for (int g = 0; g < kSteps; ++g) f.off[g] = uint32_t(16 * slot(p0, 2 * g + h));
        return f;
    }
    // fragment(lds, p0 + 32 i, g, h), from the lane's offsets.
    __device__ static __forceinline__ v8bf fragment(const char *lds, const Lane &f, int i, int g)
    {
        return *reinterpret_cast<const v8bf *>(lds + f.off[g] + i * 32 * kRowBytes);
    }
};

template <class Cfg, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::threads, Cfg::threads))) void
packed_kernel(int M, int N, int K, const u16 *__restrict__ A, int64_t lda, const u16 *__restrict__ B,
              int64_t ldb, float *__restrict__ C, int64_t ldc, int tiles_m, int tiles_n, int tile_base,
              int dma_ok)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
    using TA = Tile<Cfg, BM>;
    using TB = Tile<Cfg, BN>;
    constexpr int kStage = TA::bytes + TB::bytes;
    __shared__ __attribute__((aligned(1024))) char buf0[kStage];
    __shared__ __attribute__((aligned(1024))) char buf1[kStage];
    __shared__ __attribute__((aligned(1024))) char buf2[Cfg::nbuf > 2 ? kStage : 16];
    __shared__ __attribute__((aligned(1024))) char buf3[Cfg::nbuf > 3 ? kStage : 16];

    int tm, tn;
    tile_of<Cfg::group_m>(tile_base + int(blockIdx.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool inside = (m0 + BM <= M) && (n0 + BN <= N);
    const int wave = int(threadIdx.x) / kWave, lane = int(threadIdx.x) % kWave;
    const int wm = (wave / Cfg::waves_n) * Cfg::WM, wn = (wave % Cfg::waves_n) * Cfg::WN;
    const int half = lane / 32, l32 = lane % 32;
    const int stages = ceil_div(K, BK);
    const int full = K / BK;
    const typename TA::Lane fra = TA::lane_offsets(wm + l32, half);
    const typename TB::Lane frb = TB::lane_offsets(wn + l32, half);

    constexpr bool kChunked = Cfg::fold > 0;
    v16f acc[FM][FN], part[kChunked ? FM : 1][kChunked ? FN : 1];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{0.0f};

    // Products over the BK k values in `lds`.  Unchunked: straight into acc.
    // Chunked: into the partial tile, which FRESH starts from zero and FOLD
    // adds into acc.
    // `after_step0` runs once, after the MFMAs of the first step.
    auto compute = [&](const char *lds, auto fresh_t, auto fold_t, auto after_step0) {
        constexpr bool kFresh = decltype(fresh_t)::value;
        constexpr bool kFold = decltype(fold_t)::value;
        const char *la = lds;
        const char *lb = lds + TA::bytes;
        constexpr int kSteps = BK / 16;
        v8bf fa[2][FM], fb[2][FN];
        auto read = [&](int g, int s) {
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[s][i] = TA::fragment(la, fra, i, g);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[s][j] = TB::fragment(lb, frb, j, g);
        };
        read(0, 0);
        // Raised issue priority while this wave feeds the matrix core: the
        // scheduler then prefers waves with MFMAs to issue over waves copying
        // or waiting (S4k: 1168 vs 1136 TFLOP/s).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int g = 0; g < kSteps; ++g) {
            const int cur = g & 1;
            if (g + 1 < kSteps) read(g + 1, (g + 1) & 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (kChunked) {
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fa[cur][i], fb[cur][j], (kFresh && g == 0) ? v16f{0.0f} : part[i][j], 0, 0, 0);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j],
                                                                           acc[i][j], 0, 0, 0);
                    }
                }
            if (g == 0) after_step0();
            // Spread the next step's LDS reads between this step's MFMAs.
            if (g + 1 < kSteps) {
                constexpr int kReads = FM + FN, kMfma = FM * FN;
                constexpr int per = kMfma / kReads > 0 ? kMfma / kReads : 1;
#pragma unroll
                for (int q = 0; q < kReads; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMAs
                }
                if (kMfma > per * kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - per * kReads, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (kChunked && kFold) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j];
        }
    };

    if (VEC && dma_ok && inside && full >= 1) {
        uint32_t oa[TA::dma_per_wave], ob[TB::dma_per_wave];
#pragma unroll
        for (int q = 0; q < TA::dma_per_wave; ++q) oa[q] = TA::dma_offset(lda, wave, lane, q);
#pragma unroll
        for (int q = 0; q < TB::dma_per_wave; ++q) ob[q] = TB::dma_offset(ldb, wave, lane, q);
        const char *ga = reinterpret_cast<const char *>(A + int64_t(m0) * lda);
        const char *gb = reinterpret_cast<const char *>(B + int64_t(n0) * ldb);
#if GEMM_PACKED_BUFFER_DMA
        // the wave index in a scalar register for the copies' LDS address
        // (M0); the mask states its range, which the compiler needs to see
        // that a copy does not write the buffer being read
        static_assert((Cfg::waves & (Cfg::waves - 1)) == 0, "a power-of-two wave count");
        const int wave_s = __builtin_amdgcn_readfirstlane(wave) & (Cfg::waves - 1);
#endif
        constexpr int NB = Cfg::nbuf, FOLD = Cfg::fold;
        constexpr int D = TA::dma_per_wave + TB::dma_per_wave;  // copies per wave per stage
        auto bufp = [&](auto idx) -> char * {
            constexpr int I = decltype(idx)::value;
            return I == 0 ? buf0 : I == 1 ? buf1 : I == 2 ? buf2 : buf3;
        };
        auto dma = [&](char *lds, int st) {
#if GEMM_PACKED_BUFFER_DMA
            TA::dma_buffer(lds, ga, uint32_t(2 * BK * st), oa, wave_s);
            TB::dma_buffer(lds + TA::bytes, gb, uint32_t(2 * BK * st), ob, wave_s);
#else
            TA::dma(lds, ga + 2 * BK * st, oa, wave);
            TB::dma(lds + TA::bytes, gb + 2 * BK * st, ob, wave);
#endif
        };
        // Rings of more than two 64-k buffers keep their copies in flight
        // across the barriers (below); they issue exactly NB - 1 stages up
        // front, repeating the last one where there are fewer.  (The 1024 x
        // 4096 x 8192 weight gradient: 983-987 against 877-886 TFLOP/s; 1024^3
        // 209.4-209.6 against 204.5.  The ring of 32-k stages, which takes the
        // ragged products, measured 2.5 % slower that way and stays fenced.)
        constexpr bool kDeep = GEMM_PACKED_DEEP && NB > 2 && BK == 64;
        dma(buf0, 0);
        if (NB > 2 && (kDeep || 1 < full)) dma(bufp(Int<1 % NB>{}), min(1, full - 1));
        if (NB > 3 && (kDeep || 2 < full)) dma(bufp(Int<2 % NB>{}), min(2, full - 1));
        constexpr int TRIP = NB > FOLD ? NB : FOLD;
        if constexpr (kDeep) {
            // Each wave waits for its own copies of the stage it is about to
            // read, and the barrier is not fenced (a fence would wait for
            // every copy in flight).  Every stage issues one copy (past the
            // last stage, the last one again, into a buffer that is not
            // read), so that a count of outstanding copies names a stage;
            // whole trips have no branches, so the compiler can tell which
            // buffer each copy writes and does not wait for copies before
            // the reads.  (Copies are issued right after the barrier by
            // every wave: the stagger is for fenced rings.)
            constexpr int F = FOLD > 0 ? FOLD : 1;
            auto stage = [&](auto bi, int st) {
                constexpr int b = decltype(bi)::value;
                wait_vm<(NB - 2) * D>();              // stage st has landed
                __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS reads are done
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                dma(bufp(Int<(b + NB - 1) % NB>{}), min(st + NB - 1, full - 1));
                compute(bufp(Int<b % NB>{}), Bool<b % F == 0>{}, Bool<b % F == F - 1>{}, [] {});
            };
            int s = 0;
            for (; s + TRIP <= full; s += TRIP) unroll_for<TRIP>([&](auto bi) { stage(bi, s + decltype(bi)::value); });
            if (s < full)
                unroll_for<TRIP>([&](auto bi) {
                    if (s + decltype(bi)::value < full) stage(bi, s + decltype(bi)::value);
                });
            wait_vm<0>();
        } else if constexpr (GEMM_PACKED_RUNTIME_BUFFER && NB == 2 && FOLD == 0 && !Cfg::stagger) {
            // One running sum in two buffers: a plain loop that picks the
            // buffer from the stage's parity, so one set of fragment
            // addresses is live instead of one per unrolled stage.
            for (int st = 0; st < full; ++st) {
                wait_vm<0>();
                __syncthreads();
                char *cur = (st & 1) ? buf1 : buf0;
                char *nxt = (st & 1) ? buf0 : buf1;
                if (st + 1 < full) dma(nxt, st + 1);
                compute(cur, Bool<true>{}, Bool<true>{}, [] {});
            }
        } else
        for (int s = 0; s < full; s += TRIP) {
            unroll_for<TRIP>([&](auto bi) {
                constexpr int b = decltype(bi)::value;
                const int st = s + b;
                if (st < full) {
                    // Stage st has landed once at most the copies of the
                    // NB - 2 later stages are outstanding; after the barrier
                    // every wave's share is visible and every wave is done
                    // with stage st - 1, whose buffer the next copy refills.
                    // (__syncthreads' release fence makes the compiler wait
                    // for all outstanding copies before the barrier anyway;
                    // a fence-less barrier that kept them in flight was
                    // measured no faster: 4096^3 1198 vs 1204 TFLOP/s.)
                    if (NB == 2 || st + NB - 2 >= full)
                        wait_vm<0>();
                    else
                        wait_vm<(NB - 2) * D>();
                    __syncthreads();
                    // Copies are counted per wave in issue order, so a wave
                    // that copies after the first step still has the same
                    // count outstanding at the next wait.
                    const bool late = Cfg::stagger && wave >= Cfg::waves / 2;
                    if (!late && st + NB - 1 < full) dma(bufp(Int<(b + NB - 1) % NB>{}), st + NB - 1);
                    constexpr int F = FOLD > 0 ? FOLD : 1;
                    compute(bufp(Int<b % NB>{}), Bool<b % F == 0>{}, Bool<b % F == F - 1>{}, [&] {
                        if (late && st + NB - 1 < full) dma(bufp(Int<(b + NB - 1) % NB>{}), st + NB - 1);
                    });
                }
            });
        }
        if (kChunked && full % (FOLD > 0 ? FOLD : 1) != 0) {  // the last chunk was cut short
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j];
        }
        __syncthreads();  // every wave is done with the last full stage's buffer
        if (full < stages) {
            v4u ra[TA::per_thread], rb[TB::per_thread];
            TA::template load<VEC>(A, lda, M, K, m0, full * BK, ra);
            TB::template load<VEC>(B, ldb, N, K, n0, full * BK, rb);
            TA::store(buf0, ra);
            TB::store(buf0 + TA::bytes, rb);
            __syncthreads();
            compute(buf0, Bool<true>{}, Bool<true>{}, [] {});
        }
    } else {
        // Register-staged: stage s + 1 is loaded while stage s is computed,
        // and written to the other buffer after it (that buffer was last read
        // in stage s - 1, finished by every wave before the barrier ending it).
        v4u ra[TA::per_thread], rb[TB::per_thread];
        TA::template load<VEC>(A, lda, M, K, m0, 0, ra);
        TB::template load<VEC>(B, ldb, N, K, n0, 0, rb);
        TA::store(buf0, ra);
        TB::store(buf0 + TA::bytes, rb);
        __syncthreads();
        for (int s = 0; s < stages; ++s) {
            char *cur = (s & 1) ? buf1 : buf0;
            char *nxt = (s & 1) ? buf0 : buf1;
            if (s + 1 < stages) {
                // nxt was released by the barrier that ended stage s - 1
                if (GEMM_LDS_POISON) {
                    TA::poison(nxt);
                    TB::poison(nxt + TA::bytes);
                    poison_wait();
                }
                TA::template load<VEC>(A, lda, M, K, m0, (s + 1) * BK, ra);
                TB::template load<VEC>(B, ldb, N, K, n0, (s + 1) * BK, rb);
            }
            compute(cur, Bool<true>{}, Bool<true>{}, [] {});
            if (s + 1 < stages) {
                TA::store(nxt, ra);
                TB::store(nxt + TA::bytes, rb);
            }
            __syncthreads();
        }
    }

    // Lane l of a 32 x 32 block holds column l % 32 and, in accumulator slot
    // v, row 8 * (v / 4) + 4 * (l / 32) + v % 4.  (Swapping the operands
    // would give each lane four consecutive columns, one 16-byte store instead
    // of four 4-byte ones, but each store instruction then covers 32 rows of
    // 32 bytes instead of 2 rows of 128: measured slower, 1084 vs 1109
    // TFLOP/s at S4k.)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn + j * kBlk + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm + i * kBlk + 8 * (v / 4) + 4 * half + (v % 4);
                // C is written once: a streaming (non-temporal) store
                // (8192 x 1024 x 4096: +1.4 %; 4096^3 unchanged).
                if (inside || (row < M && col < N))
                    __builtin_nontemporal_store(acc[i][j][v], &C[int64_t(row) * ldc + col]);
            }
        }
}

// Large: 256 x 256, 8 waves of 64 x 128, one accumulator, 64-k stages in two
// buffers (128 KB of LDS; measured against 32-k stages in a four-buffer ring
// at S4k: 1104 vs 1067 TFLOP/s, the barrier count halved mattering more
// than the deeper ring).  Mid: 256 x 128, 8 waves of 64 x 64, otherwise the
// same (96 KB), for grids with fewer large tiles than CUs (8192 x 1024 x
// 4096: 900 vs 750 TFLOP/s on the small tile, whose 32-k stages it also
// beats), with staggered copies (+3 % there; neutral on the 256 x 256 tile).  Small: 128 x 128, 8 waves of 32 x 64, 32-k stages
// in a four-buffer ring, runs of 128 k summed into a fresh partial first
// (about 100 registers, so two workgroups share a CU).
#ifndef GEMM_PACKED_LARGE_CONFIG
#define GEMM_PACKED_LARGE_CONFIG 256, 256, 64, 4, 2, 2, 4, 0
#endif
#ifndef GEMM_PACKED_MID_CONFIG
#define GEMM_PACKED_MID_CONFIG 256, 128, 64, 4, 2, 2, 4, 0, 1
#endif
#ifndef GEMM_PACKED_SMALL_CONFIG
#define GEMM_PACKED_SMALL_CONFIG 128, 128, 32, 4, 2, 4, 8, 4
#endif
// SmallDeep: the small tile with 64-k stages in a four-buffer ring, runs of
// 256 k and staggered copies, for problems whose tiles are all interior and
// whose stages are all whole (1024 x 4096 x 8192: 835-844 vs 695-702
// TFLOP/s; 1024^3: 176-186 vs 158).  The ragged 2049 x 3071 x 769 product
// stays on 32-k stages (349 vs 292-295): its partial last stage and its
// register-staged edge tiles cost more with deeper stages.
#ifndef GEMM_PACKED_SMALL_DEEP_CONFIG
#define GEMM_PACKED_SMALL_DEEP_CONFIG 128, 128, 64, 4, 2, 4, 8, 4, 1
#endif
using Large = Config<GEMM_PACKED_LARGE_CONFIG>;
using Mid = Config<GEMM_PACKED_MID_CONFIG>;
using Small = Config<GEMM_PACKED_SMALL_CONFIG>;
using SmallDeep = Config<GEMM_PACKED_SMALL_DEEP_CONFIG>;
static_assert(SmallDeep::BM == Small::BM && SmallDeep::BN == Small::BN, "one small tile, two stage depths");

// The large tile from one tile per CU: below that (e.g. 8192 x 1024, 128
// large tiles) half the CUs would idle, and 128 x 128 tiles are faster
// (749 vs 682 TFLOP/s).
#ifndef GEMM_PACKED_LARGE_FROM
#define GEMM_PACKED_LARGE_FROM 256
#endif
constexpr int kLargeMaxK = 16384;  // beyond this an unchunked sum drifts towards the 1e-6 bound

template <class Cfg>
void dispatch(const PackedProblem &p, hipStream_t s)
{
    const int tiles_m = ceil_div(p.M, Cfg::BM), tiles_n = ceil_div(p.N, Cfg::BN);
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    const bool vec = reinterpret_cast<uintptr_t>(p.A) % 16 == 0 && reinterpret_cast<uintptr_t>(p.B) % 16 == 0 &&
                     p.lda % 8 == 0 && p.ldb % 8 == 0;
    // The DMA offsets are 32-bit byte offsets from a tile's first row, to
    // which the stage's offset along k (less than one row) is added.
    const int dma_ok = int64_t(Cfg::BM + 1) * p.lda * 2 < (int64_t(1) << 32) &&
                       int64_t(Cfg::BN + 1) * p.ldb * 2 < (int64_t(1) << 32);
    for (int64_t base = 0; base < tiles; base += kMaxGrid) {
        const int64_t n = tiles - base < kMaxGrid ? tiles - base : kMaxGrid;
        if (vec)
            packed_kernel<Cfg, true><<<dim3(unsigned(n)), dim3(Cfg::threads), 0, s>>>(
                p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, int(base), dma_ok);
        else
            packed_kernel<Cfg, false><<<dim3(unsigned(n)), dim3(Cfg::threads), 0, s>>>(
                p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, int(base), 0);
    }
}

// ------------------------------------------------------------- packing ---

constexpr int kPackThreads = 256;
constexpr int kPackTile = 64;  // transposing pack: 64 x 64 tiles through LDS

__device__ __forceinline__ u16 bf16_bits(float x)
{
    return __builtin_bit_cast(u16, __bf16(x));  // v_cvt_pk_bf16_f32: nearest, ties to even
}

// dst[r][c] = bf16(src[r][c]).  Workgroup (x, y) rounds columns
// [x * kRowChunk, +kRowChunk) of rows y, y + gridDim.y, ...: each lane takes
// four groups of four consecutive columns kPackThreads groups apart, so a
// wave reads 1 KB contiguous per load and each lane has four loads in
// flight.  VEC: 16-byte source and 8-byte destination vectors are aligned.
constexpr int kRowUnroll = 4;
constexpr int kRowChunk = 4 * kPackThreads * kRowUnroll;  // columns per workgroup

template <bool VEC>
__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(int rows, int cols, const float *__restrict__ src,
                                                                 int64_t lds, u16 *__restrict__ dst, int64_t ldd)
{
    const int64_t c0 = int64_t(blockIdx.x) * kRowChunk + 4 * int(threadIdx.x);  // cols may approach 2^31
    for (int r = blockIdx.y; r < rows; r += gridDim.y) {
        const float *s = src + int64_t(r) * lds;
        u16 *d = dst + int64_t(r) * ldd;
        v4f x[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int64_t c = c0 + 4 * kPackThreads * u;
            if (VEC && c + 3 < cols) {
                x[u] = *reinterpret_cast<const v4f *>(s + c);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[u][e] = (c + e < cols) ? s[c + e] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int64_t c = c0 + 4 * kPackThreads * u;
            if (VEC && c + 3 < cols) {
                const unsigned lo = unsigned(bf16_bits(x[u][0])) | (unsigned(bf16_bits(x[u][1])) << 16);
                const unsigned hi = unsigned(bf16_bits(x[u][2])) | (unsigned(bf16_bits(x[u][3])) << 16);
                *reinterpret_cast<v2u *>(d + c) = v2u{lo, hi};
            } else {
                for (int e = 0; e < 4 && c + e < cols; ++e) d[c + e] = bf16_bits(x[u][e]);
            }
        }
    }
}

// dst[r][c] = bf16(src[c][r]) (src stored cols x rows): 64 x 64 tiles read
// along the rows of src and written along the rows of dst, transposed
// through an LDS tile padded by one float per row.
template <bool VEC>
__global__ __launch_bounds__(kPackThreads) void pack_transposed_kernel(int rows, int cols,
                                                                       const float *__restrict__ src, int64_t lds,
                                                                       u16 *__restrict__ dst, int64_t ldd)
{
    __shared__ float tile[kPackTile][kPackTile + 1];
    const int tr = (rows + kPackTile - 1) / kPackTile, tc = (cols + kPackTile - 1) / kPackTile;
    const int64_t tiles = int64_t(tr) * tc;
    const int t = int(threadIdx.x);
    const int sub = t / 16, quad = 4 * (t % 16);  // 16 lanes per 64-wide row, 16 rows per pass
    for (int64_t b = blockIdx.x; b < tiles; b += gridDim.x) {
        const int r0 = int(b % tr) * kPackTile, c0 = int(b / tr) * kPackTile;
        // tile[i][j] = src[c0 + i][r0 + j]
#pragma unroll
        for (int pass = 0; pass < kPackTile / 16; ++pass) {
            const int i = sub + 16 * pass;
            const int c = c0 + i, r = r0 + quad;
            const float *s = src + int64_t(c) * lds + r;
            v4f x = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            if (c < cols) {
                if (VEC && r + 3 < rows) {
                    x = *reinterpret_cast<const v4f *>(s);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (r + e < rows) ? s[e] : 0.0f;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[i][quad + e] = x[e];
        }
        __syncthreads();
        // dst[r0 + j][c0 + quad .. +3] = tile[quad .. +3][j]
#pragma unroll
        for (int pass = 0; pass < kPackTile / 16; ++pass) {
            const int j = sub + 16 * pass;
            const int r = r0 + j, c = c0 + quad;
            if (r < rows) {
                u16 *d = dst + int64_t(r) * ldd + c;
                if (VEC && c + 3 < cols) {
                    const unsigned lo = unsigned(bf16_bits(tile[quad][j])) | (unsigned(bf16_bits(tile[quad + 1][j])) << 16);
                    const unsigned hi = unsigned(bf16_bits(tile[quad + 2][j])) | (unsigned(bf16_bits(tile[quad + 3][j])) << 16);
                    *reinterpret_cast<v2u *>(d) = v2u{lo, hi};
                } else {
                    for (int e = 0; e < 4 && c + e < cols; ++e) d[e] = bf16_bits(tile[quad + e][j]);
                }
            }
        }
        __syncthreads();  // the tile is rewritten by the next iteration
    }
}

}  // namespace

hipError_t launch_bf16_packed(const PackedProblem &p, hipStream_t s, int tile)
{
    // The largest tile that still gives every CU a tile of its own (and
    // wastes at most a quarter of its area past the edges of C).
    auto tiles = [&](int bm, int bn) { return int64_t(ceil_div(p.M, bm)) * ceil_div(p.N, bn); };
    auto fits = [&](int bm, int bn) { return 4 * int64_t(p.M) * p.N >= 3 * tiles(bm, bn) * bm * bn; };
    if (tile == 0) {
        if (p.K > kLargeMaxK)
            tile = Small::BM * Small::BN;
        else if (tiles(Large::BM, Large::BN) >= GEMM_PACKED_LARGE_FROM && fits(Large::BM, Large::BN))
            tile = Large::BM * Large::BN;
        else if (tiles(Mid::BM, Mid::BN) >= GEMM_PACKED_LARGE_FROM && fits(Mid::BM, Mid::BN))
            tile = Mid::BM * Mid::BN;
        else
            tile = Small::BM * Small::BN;
    }
    if (tile == Large::BM * Large::BN && p.K <= kLargeMaxK)
        dispatch<Large>(p, s);
    else if (tile == Mid::BM * Mid::BN && p.K <= kLargeMaxK)
        dispatch<Mid>(p, s);
    else if (p.M % SmallDeep::BM == 0 && p.N % SmallDeep::BN == 0 && p.K % SmallDeep::BK == 0)
        dispatch<SmallDeep>(p, s);
    else
        dispatch<Small>(p, s);
    return hipGetLastError();
}

hipError_t launch_pack_bf16(int rows, int cols, const float *src, int64_t lds, int trans, uint16_t *dst,
                            int64_t ldd, hipStream_t s)
{
    const bool src_vec = reinterpret_cast<uintptr_t>(src) % 16 == 0 && lds % 4 == 0;
    const bool dst_vec = reinterpret_cast<uintptr_t>(dst) % 8 == 0 && ldd % 4 == 0;
    const bool vec = src_vec && dst_vec;
    // A grid of up to 64 workgroups per CU's worth; the kernels stride over the rest.
    constexpr int64_t kMaxBlocks = 256 * 64;
    if (!trans) {
        // x: column chunks (at most 2^31 / kRowChunk); y: rows, strided
        // beyond the grid's y limit, and capped so that about kMaxBlocks
        // workgroups are launched in all.
        const int64_t gx = (int64_t(cols) + kRowChunk - 1) / kRowChunk;
        int64_t gy = kMaxBlocks / gx;
        gy = gy < 1 ? 1 : gy > rows ? rows : gy > kMaxGridY ? kMaxGridY : gy;
        const dim3 grid{unsigned(gx), unsigned(gy), 1u};
        if (vec)
            pack_rows_kernel<true><<<grid, dim3(kPackThreads), 0, s>>>(rows, cols, src, lds, dst, ldd);
        else
            pack_rows_kernel<false><<<grid, dim3(kPackThreads), 0, s>>>(rows, cols, src, lds, dst, ldd);
    } else {
        const int64_t tiles = int64_t((rows + kPackTile - 1) / kPackTile) * ((cols + kPackTile - 1) / kPackTile);
        const int64_t blocks = tiles < kMaxBlocks ? tiles : kMaxBlocks;
        if (vec)
            pack_transposed_kernel<true><<<dim3(unsigned(blocks)), dim3(kPackThreads), 0, s>>>(rows, cols, src, lds, dst, ldd);
        else
            pack_transposed_kernel<false><<<dim3(unsigned(blocks)), dim3(kPackThreads), 0, s>>>(rows, cols, src, lds, dst, ldd);
    }
    return hipGetLastError();
}

}  // namespace gemmf32
