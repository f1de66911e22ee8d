// tile_common.hpp -- device helpers shared by the LDS-tiled kernels (MFMA
// and vector-FMA): the operand view, the coalesced global -> register
// slice loader with zero-filled edges, and the XCD-aware tile order.
#pragma once

#include "gemm_internal.hpp"

namespace gemmf32 {

typedef float v4f __attribute__((ext_vector_type(4)));

// One operand as stored in global memory: a rows_total x cols_total
// row-major matrix with leading dimension ld.  For A untransposed the rows
// are m and the columns k; transposed, the rows are k and the columns m
// (likewise for B with n).
struct Operand {
    const float *base;
    int64_t ld;
    int rows_total, cols_total;
};

// A ROWS x COLS slice of an operand, read as 16-byte vectors along the
// contiguous direction.  Vector v of the slice (row v / (COLS/4), columns
// 4 * (v % (COLS/4)) .. +3) is handled by thread v % THREADS, as the
// per-thread index q = v / THREADS.  Consecutive threads therefore read
// consecutive 16-byte pieces of a row: a 64-lane wave reads whole rows.
template <int ROWS, int COLS, int THREADS>
struct Slice {
    static constexpr int vec_per_row = COLS / 4;
    static constexpr int vecs = ROWS * vec_per_row;
    static constexpr int per_thread = (vecs + THREADS - 1) / THREADS;
    static_assert(COLS % 4 == 0, "slice rows are whole vectors");
    static_assert(vecs % THREADS == 0 || THREADS % vecs == 0,
                  "a slice splits evenly over the block, or covers part of it");

    // tid: the thread's index in the block (threadIdx.x, or the same value
    // derived afresh where the caller wants it recomputed rather than kept).
    __device__ static __forceinline__ int index(int q, int tid) { return tid + THREADS * q; }
    // False only for the threads past the end of a slice smaller than the block.
    __device__ static __forceinline__ bool active(int q, int tid) { return vecs % THREADS == 0 || index(q, tid) < vecs; }
    __device__ static __forceinline__ int row(int q, int tid) { return index(q, tid) / vec_per_row; }
    __device__ static __forceinline__ int col(int q, int tid) { return (index(q, tid) % vec_per_row) * 4; }
    __device__ static __forceinline__ bool active(int q) { return active(q, int(threadIdx.x)); }
    __device__ static __forceinline__ int row(int q) { return row(q, int(threadIdx.x)); }
    __device__ static __forceinline__ int col(int q) { return col(q, int(threadIdx.x)); }

    // Load the slice whose stored origin is (r0, c0).  CHECK: elements
    // outside rows_total x cols_total read as zero and are never
    // dereferenced.  VEC: the operand allows aligned 16-byte loads
    // (vec4_ok); otherwise each element is loaded on its own.
    template <bool CHECK, bool VEC>
    __device__ static __forceinline__ void load(const Operand &op, int r0, int c0, v4f (&reg)[per_thread])
    {
        load<CHECK, VEC>(op, r0, c0, reg, int(threadIdx.x));
    }
    template <bool CHECK, bool VEC>
    __device__ static __forceinline__ void load(const Operand &op, int r0, int c0, v4f (&reg)[per_thread],
                                                int tid)
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            if (!active(q, tid)) {
                reg[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                continue;
            }
            const int r = r0 + row(q, tid);
            const int c = c0 + col(q, tid);
            const float *src = op.base + int64_t(r) * op.ld + c;
            if (!CHECK) {
                if (VEC) {
                    reg[q] = *reinterpret_cast<const v4f *>(src);
                } else {
                    reg[q] = v4f{src[0], src[1], src[2], src[3]};
                }
            } else {
                const bool row_ok = r < op.rows_total;
                if (VEC && row_ok && c + 3 < op.cols_total) {
                    reg[q] = *reinterpret_cast<const v4f *>(src);
                } else {
                    v4f x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (row_ok && c + e < op.cols_total) ? src[e] : 0.0f;
                    reg[q] = x;
                }
            }
        }
    }
};

constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kCUs = 256;  // MI355X: compute units (32 per XCD)

// Wait until at most N of this wave's vector-memory operations (here: the
// global -> LDS copies) are outstanding; they complete in issue order.
// gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8
// left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One 16-byte global -> LDS copy per lane: lane l's vector at byte offset
// off from base (wave-uniform) lands at lds_piece + 16 l bytes.  Issued as a
// buffer load on a raw descriptor of base (no stride, no range limit: the
// host keeps every offset below 2^32; the data format untyped loads need on
// this family), so a lane keeps only its 32-bit offset; GEMM_BUFFER_DMA 0
// issues global_load_lds with a 64-bit address per lane instead.
#ifndef GEMM_BUFFER_DMA
#define GEMM_BUFFER_DMA 1
#endif
//
// `avail` is the number of bytes from base to the end of the operand's
// storage: the hardware's range check then turns a lane whose vector lies
// past it into a read of zeros instead of a read past the allocation (edge
// tiles copy whole stages; the rows or columns outside the matrix only feed
// outputs that are never stored).
__device__ __forceinline__ void copy16_to_lds(float *lds_piece, const char *base, uint32_t off,
                                              uint32_t avail = 0xFFFFFFFFu)
{
    if (GEMM_BUFFER_DMA) {
        const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), short(0), int(avail),
                                                            int(0x00020000));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_piece, 16, off, 0,
                                                 0, 0);
    } else {
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const float *>(base + off), lds_piece, 16, 0, 0);
    }
}

// GEMM_LDS_POISON 1 builds the race-detection ablation (the library is built
// with 0): before a stage buffer is refilled, each lane first writes NaN
// over exactly the LDS bytes its own copies (or stores) of the refill will
// fill, and waits until those writes are done.  The buffer then holds NaN
// from the moment the barrier releases it until the refill lands, so a wave
// that reads it too early (a missing wait) or still reads the previous
// stage after the release (a missing barrier) multiplies NaN, which reaches
// C.  Results are otherwise unchanged.
#ifndef GEMM_LDS_POISON
#define GEMM_LDS_POISON 0
#endif

// Write NaN over the 16 bytes at `lds` (poison build only).
__device__ __forceinline__ void poison16(void *lds)
{
    if (GEMM_LDS_POISON) {
        const float q = __builtin_nanf("");
        *reinterpret_cast<v4f *>(lds) = v4f{q, q, q, q};
    }
}
// Wait until this wave's LDS writes are done (poison build only): vmcnt and
// expcnt left at their maxima, lgkmcnt 0.
__device__ __forceinline__ void poison_wait()
{
    if (GEMM_LDS_POISON) __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Workgroup index -> (tile row, tile column) of a tiles_m x tiles_n grid.
// Step 1 inverts the round-robin dealing of consecutive workgroups to the
// XCDs, so that XCD x owns one contiguous range of the remapped index w.
// Step 2 walks w GROUP_M tile-rows at a time, down each column of the
// group before moving right, so the workgroups resident on one XCD at the
// same time cover a compact block of C and share A and B panels in its L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int tiles = tiles_m * tiles_n;
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    const int w = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
    const int per_group = GROUP_M * tiles_n;
    const int first = (w / per_group) * GROUP_M;
    const int gm = min(tiles_m - first, GROUP_M);
    const int local = w % per_group;
    tm = first + local % gm;
    tn = local / gm;
}

constexpr int kMaxGrid = 1 << 20;  // grid x cap; larger grids are split (or strided over)
constexpr int kMaxGridY = 65535;   // grid y cap (batched products)

}  // namespace gemmf32
