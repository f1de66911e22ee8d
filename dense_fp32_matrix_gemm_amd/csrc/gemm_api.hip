// gemm_api.hip -- the C ABI of the FP32 GEMM library: argument validation,
// kernel selection and launch-error mapping.  Contract: include/gemm_f32.h.
//
// Validation happens entirely on the host, before any HIP call, so invalid
// arguments are reported with the same codes on a machine without a GPU.
#include "gemm_f32.h"
#include "gemm_internal.hpp"

#include <climits>
#include <mutex>

namespace {

using gemmf32::Problem;

constexpr int64_t kDimLimit = int64_t(INT_MAX);  // dimensions are < 2^31

// Argument positions (1-based) as in the prototypes, for the -i codes.
enum Arg {
    kArgM = 1, kArgN, kArgK, kArgA, kArgLda, kArgB, kArgLdb, kArgC, kArgLdc,
    kArgTransA, kArgTransB, kArgStream, kArgAlgo
};

// check_ptrs false: nothing will be read or written (an empty batch), so
// the pointers may be anything.
int validate(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
             const float *B, int64_t ldb, const float *C, int64_t ldc,
             int transA, int transB, bool check_ptrs = true)
{
    if (M < 0 || M > kDimLimit) return -kArgM;
    if (N < 0 || N > kDimLimit) return -kArgN;
    if (K < 0 || K > kDimLimit) return -kArgK;
    if (transA != 0 && transA != 1) return -kArgTransA;
    if (transB != 0 && transB != 1) return -kArgTransB;
    const int64_t a_row = transA ? M : K;   // length of a stored row of A
    const int64_t b_row = transB ? K : N;   // length of a stored row of B
    if (check_ptrs && A == nullptr && M * K > 0) return -kArgA;
    if (lda < (a_row > 1 ? a_row : 1) || lda > kDimLimit) return -kArgLda;
    if (check_ptrs && B == nullptr && K * N > 0) return -kArgB;
    if (ldb < (b_row > 1 ? b_row : 1) || ldb > kDimLimit) return -kArgLdb;
    if (check_ptrs && C == nullptr && M * N > 0) return -kArgC;
    if (ldc < (N > 1 ? N : 1) || ldc > kDimLimit) return -kArgLdc;
    return 0;
}

// Split k: runs of len = ceil(K / splits) rounded up to whole 32-k stages,
// and the number of non-empty runs that gives (K, splits >= 1).
int64_t splitk_len(int64_t K, int64_t splits)
{
    const int64_t per = (K + splits - 1) / splits;
    return (per + 31) / 32 * 32;
}
int64_t splitk_used(int64_t K, int64_t splits)
{
    const int64_t len = splitk_len(K, splits);
    return (K + len - 1) / len;
}

// Device memory of gemm_f32_splitk_noalloc: the split-k partial products of
// callers that cannot allocate.  Each GPU the library runs on holds its own
// copy until the process ends, and every call on that GPU shares it.  In
// host code `scratch` names a host-side stand-in, never the device array:
// host code uses only the address hipGetSymbolAddress returns for it.
static __device__ __align__(256) float scratch[GEMM_F32_SPLITK_SCRATCH_BYTES / 4];

constexpr int kMaxDevices = 64;
std::mutex scratch_lock;
float *scratch_addr[kMaxDevices];  // per device, filled on its first call

// The device address of `scratch` on the GPU that runs `stream` (the
// current device for the null stream), looked up once per device with that
// device current.
hipError_t scratch_on(hipStream_t stream, float **out)
{
    int dev = 0;
    hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(scratch_lock);
    if (scratch_addr[dev] == nullptr) {
        int cur = 0;
        if ((err = hipGetDevice(&cur)) != hipSuccess) return err;
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void *addr = nullptr;
        err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        if (addr == nullptr) return hipErrorInvalidSymbol;
        scratch_addr[dev] = static_cast<float *>(addr);
    }
    *out = scratch_addr[dev];
    return hipSuccess;
}

// The split-k launches for a validated problem with s_used > 1: the partial
// products into ws (s_used packed M x N slices), then their fixed-order sum
// into C.
hipError_t launch_splitk(Problem p, int64_t K, int64_t splits, float *ws, hipStream_t s)
{
    // Partial s reads op(A)[:, s*len ..] and op(B)[s*len .., :]: a run of k
    // moves along the stored rows of an operand whose rows hold k (A
    // untransposed, B transposed), else down its rows.
    float *C = p.C;
    const int64_t ldc = p.ldc;
    const int64_t len = splitk_len(K, splits);
    const int64_t used = splitk_used(K, splits);
    p.K = int(len);
    p.k_total = int(K);
    p.stride_a = p.transA ? len * p.lda : len;
    p.stride_b = p.transB ? len : len * p.ldb;
    p.C = ws;
    p.ldc = p.N;
    p.stride_c = int64_t(p.M) * p.N;
    p.batch = used;
    hipError_t err = gemmf32::launch_mfma(p, s, 0);
    if (err == hipSuccess) err = gemmf32::launch_splitk_reduce(ws, int(used), p.M, p.N, C, ldc, s);
    return err;
}

int run(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
        const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
        int transB, void *stream, int algo)
{
    const int bad = validate(M, N, K, A, lda, B, ldb, C, ldc, transA, transB);
    if (bad) return bad;
    if (algo < GEMM_F32_ALGO_AUTO || algo > GEMM_F32_ALGO_MFMA_WIDE) return -kArgAlgo;
    const Problem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc, transA, transB};
    // The 256 x 256 kernel runs only the problems in its domain.
    if (algo == GEMM_F32_ALGO_MFMA_WIDE && M > 0 && N > 0 && K > 0 && !gemmf32::mfma_wide_fits(p))
        return -kArgAlgo;
    if (M == 0 || N == 0) return 0;  // nothing to write

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (K == 0) {
        err = gemmf32::launch_zero_fill(p, s);
    } else {
        switch (algo) {
        case GEMM_F32_ALGO_NAIVE: err = gemmf32::launch_naive(p, s); break;
        case GEMM_F32_ALGO_TILED: err = gemmf32::launch_tiled(p, s); break;
        case GEMM_F32_ALGO_FMA: err = gemmf32::launch_fma(p, s); break;
        case GEMM_F32_ALGO_MFMA_TILE128: err = gemmf32::launch_mfma(p, s, 128); break;
        case GEMM_F32_ALGO_MFMA_TILE64: err = gemmf32::launch_mfma(p, s, 64); break;
        case GEMM_F32_ALGO_MFMA_TILE256: err = gemmf32::launch_mfma(p, s, 256); break;
        case GEMM_F32_ALGO_MFMA_WIDE: err = gemmf32::launch_mfma_wide(p, s); break;
        case GEMM_F32_ALGO_MFMA:
        case GEMM_F32_ALGO_AUTO:
        default: err = gemmf32::launch_mfma(p, s, 0); break;
        }
    }
    return err == hipSuccess ? 0 : int(err);
}

}  // namespace

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
             const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
             int transB, void *stream)
{
    return run(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream,
               GEMM_F32_ALGO_AUTO);
}

int gemm_f32_naive(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                   const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
                   int transB, void *stream)
{
    return run(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream,
               GEMM_F32_ALGO_NAIVE);
}

int gemm_f32_ex(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
                int transB, void *stream, int algo)
{
    return run(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream, algo);
}

const char *gemm_f32_strerror(int status)
{
    switch (status) {
    case 0: return "success";
    case -kArgM: return "invalid argument 1 (M): negative or >= 2^31";
    case -kArgN: return "invalid argument 2 (N): negative or >= 2^31";
    case -kArgK: return "invalid argument 3 (K): negative or >= 2^31";
    case -kArgA: return "invalid argument 4 (A): NULL with M*K > 0";
    case -kArgLda: return "invalid argument 5 (lda): smaller than a stored row of A, or >= 2^31";
    case -kArgB: return "invalid argument 6 (B): NULL with K*N > 0";
    case -kArgLdb: return "invalid argument 7 (ldb): smaller than a stored row of B, or >= 2^31";
    case -kArgC: return "invalid argument 8 (C): NULL with M*N > 0";
    case -kArgLdc: return "invalid argument 9 (ldc): smaller than N, or >= 2^31";
    case -kArgTransA: return "invalid argument 10 (transA): not 0 or 1";
    case -kArgTransB: return "invalid argument 11 (transB): not 0 or 1";
    case -12: return "invalid argument 12 (gemm_f32_splitk: splits < 1 or too large a workspace; "
                     "gemm_f32_splitk_noalloc: the same, or partial products larger than "
                     "GEMM_F32_SPLITK_SCRATCH_BYTES (use fewer splits); "
                     "gemm_f32_strided_batched: strideC negative or overlapping)";
    case -kArgAlgo: return "invalid argument 13 (gemm_f32_ex: unknown kernel family; gemm_f32_bias_act: "
                           "unknown activation; gemm_f32_splitk: workspace NULL; "
                           "gemm_f32_strided_batched: batch out of range)";
    case -14: return "invalid argument 14 (gemm_f32_splitk: workspace_bytes below the size needed; "
                     "gemm_f32_strided_batched: transA not 0 or 1)";
    case -15: return "invalid argument 15 (gemm_f32_strided_batched: transB not 0 or 1)";
    default: break;
    }
    if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}

int gemm_f32_strided_batched(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                             int64_t strideA, const float *B, int64_t ldb, int64_t strideB,
                             float *C, int64_t ldc, int64_t strideC, int64_t batch,
                             int transA, int transB, void *stream)
{
    // Argument positions of this prototype, for the -i codes.
    enum { bM = 1, bN, bK, bA, bLda, bStrideA, bB, bLdb, bStrideB, bC, bLdc, bStrideC, bBatch,
           bTransA, bTransB };
    const int bad = validate(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, batch != 0);
    if (bad) {
        // validate() numbers the arguments as gemm_f32 does; map to this prototype
        static const int map[] = {0, bM, bN, bK, bA, bLda, bB, bLdb, bC, bLdc, bTransA, bTransB};
        return -map[-bad];
    }
    if (batch < 0 || batch > kDimLimit) return -bBatch;
    if (strideA < 0) return -bStrideA;
    if (strideB < 0) return -bStrideB;
    // Products must not write over each other: C_b spans (M-1)*ldc + N floats.
    if (strideC < 0 || (batch > 1 && M > 0 && N > 0 && strideC < (M - 1) * ldc + N)) return -bStrideC;
    if (batch == 0 || M == 0 || N == 0) return 0;
    Problem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc, transA, transB};
    p.stride_a = strideA;
    p.stride_b = strideB;
    p.stride_c = strideC;
    p.batch = batch;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = K == 0 ? gemmf32::launch_zero_fill(p, s) : gemmf32::launch_mfma(p, s, 0);
    return err == hipSuccess ? 0 : int(err);
}

int gemm_f32_bias_act(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                      const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
                      int transB, const float *bias, int act, void *stream)
{
    const int bad = validate(M, N, K, A, lda, B, ldb, C, ldc, transA, transB);
    if (bad) return bad;
    if (act != GEMM_F32_ACT_NONE && act != GEMM_F32_ACT_GELU) return -13;
    if (M == 0 || N == 0) return 0;
    Problem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc, transA, transB};
    p.bias = bias;
    p.act = act;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (K == 0)  // the empty product is 0: C = act(bias) (or act(0))
        err = gemmf32::launch_zero_fill(p, s);
    else
        err = gemmf32::launch_mfma(p, s, 0);
    return err == hipSuccess ? 0 : int(err);
}

int gemm_f32_bf16(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                  const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
                  int transB, void *stream)
{
    const int bad = validate(M, N, K, A, lda, B, ldb, C, ldc, transA, transB);
    if (bad) return bad;
    if (M == 0 || N == 0) return 0;
    const Problem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc, transA, transB};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = K == 0 ? gemmf32::launch_zero_fill(p, s) : gemmf32::launch_bf16(p, s);
    return err == hipSuccess ? 0 : int(err);
}

int gemm_f32_pack_bf16(int64_t rows, int64_t cols, const float *src, int64_t lds, int trans,
                       uint16_t *dst, int64_t ldd, void *stream)
{
    if (rows < 0 || rows > kDimLimit) return -1;
    if (cols < 0 || cols > kDimLimit) return -2;
    if (src == nullptr && rows * cols > 0) return -3;
    if (trans != 0 && trans != 1) return -5;
    const int64_t src_row = trans ? rows : cols;  // length of a stored row of src
    if (lds < (src_row > 1 ? src_row : 1) || lds > kDimLimit) return -4;
    if (dst == nullptr && rows * cols > 0) return -6;
    if (ldd < (cols > 1 ? cols : 1) || ldd > kDimLimit) return -7;
    if (rows == 0 || cols == 0) return 0;
    const hipError_t err = gemmf32::launch_pack_bf16(int(rows), int(cols), src, lds, trans, dst, ldd,
                                                     static_cast<hipStream_t>(stream));
    return err == hipSuccess ? 0 : int(err);
}

int gemm_f32_bf16_packed(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    if (M < 0 || M > kDimLimit) return -kArgM;
    if (N < 0 || N > kDimLimit) return -kArgN;
    if (K < 0 || K > kDimLimit) return -kArgK;
    if (A == nullptr && M * K > 0) return -kArgA;
    if (lda < (K > 1 ? K : 1) || lda > kDimLimit) return -kArgLda;
    if (B == nullptr && N * K > 0) return -kArgB;
    if (ldb < (K > 1 ? K : 1) || ldb > kDimLimit) return -kArgLdb;
    if (C == nullptr && M * N > 0) return -kArgC;
    if (ldc < (N > 1 ? N : 1) || ldc > kDimLimit) return -kArgLdc;
    if (M == 0 || N == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (K == 0) {
        const Problem z{int(M), int(N), 0, nullptr, 1, nullptr, 1, C, ldc, 0, 0};
        err = gemmf32::launch_zero_fill(z, s);
    } else {
        const gemmf32::PackedProblem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc};
        err = gemmf32::launch_bf16_packed(p, s);
    }
    return err == hipSuccess ? 0 : int(err);
}

int64_t gemm_f32_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int64_t splits)
{
    if (M < 0 || M > kDimLimit) return -1;
    if (N < 0 || N > kDimLimit) return -2;
    if (K < 0 || K > kDimLimit) return -3;
    if (splits < 1 || splits > kDimLimit) return -12;
    if (M == 0 || N == 0 || K == 0) return 0;
    const int64_t used = splitk_used(K, splits);
    if (used == 1) return 0;
    if (M * N > (int64_t(1) << 60) / used) return -12;  // s_used * M * N * 4 < 2^62
    return used * M * N * 4;
}

int gemm_f32_splitk(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                    const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
                    int transB, int64_t splits, float *workspace, int64_t workspace_bytes,
                    void *stream)
{
    const int bad = validate(M, N, K, A, lda, B, ldb, C, ldc, transA, transB);
    if (bad) return bad;
    const int64_t need = gemm_f32_splitk_workspace_size(M, N, K, splits);
    if (need < 0) return int(need);
    if (need > 0 && workspace == nullptr) return -13;
    if (workspace_bytes < need) return -14;
    if (M == 0 || N == 0) return 0;
    Problem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc, transA, transB};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) {
        const hipError_t err = gemmf32::launch_zero_fill(p, s);
        return err == hipSuccess ? 0 : int(err);
    }
    if (need == 0) {
        const hipError_t err = gemmf32::launch_mfma(p, s, 0);
        return err == hipSuccess ? 0 : int(err);
    }
    const hipError_t err = launch_splitk(p, K, splits, workspace, s);
    return err == hipSuccess ? 0 : int(err);
}

int gemm_f32_splitk_noalloc(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                            const float *B, int64_t ldb, float *C, int64_t ldc, int transA,
                            int transB, int64_t splits, void *stream)
{
    const int bad = validate(M, N, K, A, lda, B, ldb, C, ldc, transA, transB);
    if (bad) return bad;
    const int64_t need = gemm_f32_splitk_workspace_size(M, N, K, splits);
    if (need < 0) return int(need);
    if (need > GEMM_F32_SPLITK_SCRATCH_BYTES) return -12;  // more partials than the scratch holds
    if (M == 0 || N == 0) return 0;
    const Problem p{int(M), int(N), int(K), A, lda, B, ldb, C, ldc, transA, transB};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (K == 0) {
        err = gemmf32::launch_zero_fill(p, s);
    } else if (need == 0) {
        err = gemmf32::launch_mfma(p, s, 0);
    } else {
        // Every element of each partial is written before the sum reads it,
        // so the scratch needs no clearing between calls.
        float *ws = nullptr;
        err = scratch_on(s, &ws);
        if (err == hipSuccess) err = launch_splitk(p, K, splits, ws, s);
    }
    return err == hipSuccess ? 0 : int(err);
}

int gemm_f32_plan(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                  int64_t ldb, int64_t ldc, int transA, int transB, int64_t strideA,
                  int64_t strideB, int64_t batch)
{
    // gemm_f32's checks without the pointer checks; its ldc and transpose
    // positions (-9, -10, -11) are one place earlier in this prototype.
    const int bad = validate(M, N, K, A, lda, B, ldb, nullptr, ldc, transA, transB, false);
    if (bad) return bad <= -9 ? bad + 1 : bad;
    if (strideA < 0) return -11;
    if (strideB < 0) return -12;
    if (batch < 1 || batch > kDimLimit) return -13;
    if (M == 0 || N == 0) return GEMM_F32_PLAN_NOTHING;
    if (K == 0) return GEMM_F32_PLAN_ZERO_FILL;
    Problem p{int(M), int(N), int(K), A, lda, B, ldb, nullptr, ldc, transA, transB};
    p.stride_a = batch > 1 ? strideA : 0;
    p.stride_b = batch > 1 ? strideB : 0;
    p.batch = batch;
    return gemmf32::plan_mfma(p, 0);
}

int gemm_f32_version(void) { return 10700; }

}  // extern "C"
