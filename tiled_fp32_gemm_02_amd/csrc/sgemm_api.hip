// C-ABI entry points of the fp32 GEMM library (declared in include/sgemm.h).
//
// Host work per call: validate the arguments (BLAS-style argument positions in the
// error code), take the quick returns (empty result; alpha == 0 or K == 0 leaves
// beta*C), choose a kernel configuration from the shape and alignment, and queue
// one kernel on the caller's stream. No allocation, copy or synchronisation.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>

#include "sgemm.h"
#include "sgemm_kernels.hpp"

using sgemm_impl::GemmArgs;

namespace {

enum Kind { KIND_TILE16 = 0, KIND_MFMA = 1 };

typedef hipError_t (*LaunchFn)(const GemmArgs &, int batch, bool vec, bool edge, hipStream_t);

struct Config {
    const char *name;
    Kind kind;
    int bm, bn, bk;      // workgroup tile (tile16: 16 x 16 x 16)
    int threads;         // threads per workgroup
    int group_m;         // tile rows per L2 band in the workgroup order
    LaunchFn launch;
};

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int GROUP_M>
hipError_t launch_mfma(const GemmArgs &p, int batch, bool vec, bool edge, hipStream_t s)
{
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const dim3 grid(tiles, 1, batch), block(WGM * WGN * WGK * 64);
    if (vec && !edge)
        hipLaunchKernelGGL((sgemm_impl::sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, true, false>), grid, block, 0, s, p,
                           GROUP_M);
    else if (vec)
        hipLaunchKernelGGL((sgemm_impl::sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, true, true>), grid, block, 0, s, p,
                           GROUP_M);
    else
        hipLaunchKernelGGL((sgemm_impl::sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, false, true>), grid, block, 0, s, p,
                           GROUP_M);
    return hipGetLastError();
}

hipError_t launch_tile16(const GemmArgs &p, int batch, bool, bool, hipStream_t s)
{
    const dim3 grid((p.N + 15) / 16, (p.M + 15) / 16, batch), block(16, 16);
    hipLaunchKernelGGL(sgemm_impl::sgemm_tile16, grid, block, 0, s, p);
    return hipGetLastError();
}

// Configuration table. Ids are stable within one build; names encode the tile
// (BM x BN x BK), the wave grid (WGM x WGN) and, after "k", the wave groups along k.
const Config kConfigs[] = {
    {"tile16", KIND_TILE16, 16, 16, 16, 256, 1, launch_tile16},
    {"mfma_64x64x16_w2x2", KIND_MFMA, 64, 64, 16, 256, 8, launch_mfma<64, 64, 16, 2, 2, 1, 8>},
    {"mfma_128x128x16_w2x2", KIND_MFMA, 128, 128, 16, 256, 8, launch_mfma<128, 128, 16, 2, 2, 1, 8>},
    {"mfma_128x128x32_w2x2", KIND_MFMA, 128, 128, 32, 256, 8, launch_mfma<128, 128, 32, 2, 2, 1, 8>},
    {"mfma_256x128x16_w2x2", KIND_MFMA, 256, 128, 16, 256, 4, launch_mfma<256, 128, 16, 2, 2, 1, 4>},
    {"mfma_256x256x16_w2x4", KIND_MFMA, 256, 256, 16, 512, 4, launch_mfma<256, 256, 16, 2, 4, 1, 4>},
    {"mfma_64x64x32_w2x2", KIND_MFMA, 64, 64, 32, 256, 8, launch_mfma<64, 64, 32, 2, 2, 1, 8>},
    {"mfma_128x64x16_w2x2", KIND_MFMA, 128, 64, 16, 256, 8, launch_mfma<128, 64, 16, 2, 2, 1, 8>},
    {"mfma_64x128x16_w2x2", KIND_MFMA, 64, 128, 16, 256, 8, launch_mfma<64, 128, 16, 2, 2, 1, 8>},
    {"mfma_256x256x32_w2x4", KIND_MFMA, 256, 256, 32, 512, 4, launch_mfma<256, 256, 32, 2, 4, 1, 4>},
    {"mfma_256x128x16_w4x2", KIND_MFMA, 256, 128, 16, 512, 4, launch_mfma<256, 128, 16, 4, 2, 1, 4>},
    {"mfma_128x256x16_w2x4", KIND_MFMA, 128, 256, 16, 512, 8, launch_mfma<128, 256, 16, 2, 4, 1, 8>},
    {"mfma_128x128x32_w4x4", KIND_MFMA, 128, 128, 32, 1024, 8, launch_mfma<128, 128, 32, 4, 4, 1, 8>},
    {"mfma_64x64x16_w2x2k2", KIND_MFMA, 64, 64, 16, 512, 8, launch_mfma<64, 64, 16, 2, 2, 2, 8>},
    {"mfma_64x64x32_w2x2k2", KIND_MFMA, 64, 64, 32, 512, 8, launch_mfma<64, 64, 32, 2, 2, 2, 8>},
    {"mfma_64x64x32_w2x2k4", KIND_MFMA, 64, 64, 32, 1024, 8, launch_mfma<64, 64, 32, 2, 2, 4, 8>},
    {"mfma_64x64x64_w2x2k4", KIND_MFMA, 64, 64, 64, 1024, 8, launch_mfma<64, 64, 64, 2, 2, 4, 8>},
    {"mfma_128x64x32_w2x2k2", KIND_MFMA, 128, 64, 32, 512, 8, launch_mfma<128, 64, 32, 2, 2, 2, 8>},
    {"mfma_64x128x32_w2x2k2", KIND_MFMA, 64, 128, 32, 512, 8, launch_mfma<64, 128, 32, 2, 2, 2, 8>},
    {"mfma_128x128x32_w2x2k2", KIND_MFMA, 128, 128, 32, 512, 8, launch_mfma<128, 128, 32, 2, 2, 2, 8>},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// 128-bit path: every operand 16-byte aligned and every row start 16-byte aligned,
// and the K and N extents whole 4-float chunks (so a chunk is all in or all out).
bool vector_ok(int N, int K, const float *A, int lda, const float *B, int ldb, const float *C, int ldc)
{
    return aligned16(A) && aligned16(B) && aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 &&
           ldc % 4 == 0 && N % 4 == 0 && K % 4 == 0;
}

uint64_t tile_count(const Config &c, int M, int N)
{
    return (uint64_t)((M + c.bm - 1) / c.bm) * (uint64_t)((N + c.bn - 1) / c.bn);
}

// Auto-selection by a small cost model. A candidate's tiles spread over the 256 CUs
// take L = ceil(tiles / 256) rounds on the busiest CU; its time is L tiles of work
// (in units of one 64x64 tile) divided by the CU's throughput with that many tiles
// resident. Throughputs (fp32 TFLOP/s per CU) were measured on MI355X with the
// whole chip busy: rate_one when a CU holds a single workgroup, rate_many when it
// holds several (more waves to hide latency). The model picks the large tile when it
// fills the chip in one round and the wave-split 64x64 tile when few tiles exist;
// K cancels out because every candidate walks the same K.
struct Candidate {
    int id;
    int units;          // tile area / (64 * 64)
    double rate_one;    // per-CU rate with one resident workgroup
    double rate_many;   // per-CU rate with two or more
};

const Candidate kCandidatesVec[] = {
    {5, 16, 0.500, 0.500},    // mfma_256x256x16_w2x4: one workgroup per CU fits
    {19, 4, 0.458, 0.458},    // mfma_128x128x32_w2x2k2: one per CU
    {18, 2, 0.400, 0.452},    // mfma_64x128x32_w2x2k2: up to three per CU
    {16, 1, 0.395, 0.436},    // mfma_64x64x64_w2x2k4: up to two per CU
};
// 32-bit path (unaligned operands): the 64-deep stage loses to 32-deep ones there.
const Candidate kCandidatesScalar[] = {
    {5, 16, 0.500, 0.500},
    {19, 4, 0.458, 0.458},
    {18, 2, 0.400, 0.452},
    {14, 1, 0.380, 0.420},    // mfma_64x64x32_w2x2k2: up to four per CU
};

int choose(int M, int N, bool vec)
{
    constexpr uint64_t kCUs = 256;
    const Candidate *cands = vec ? kCandidatesVec : kCandidatesScalar;
    const int count = vec ? (int)(sizeof(kCandidatesVec) / sizeof(Candidate))
                          : (int)(sizeof(kCandidatesScalar) / sizeof(Candidate));
    int best = cands[0].id;
    double best_cost = 0.0;
    bool first = true;
    for (int i = 0; i < count; ++i) {
        const Candidate &cand = cands[i];
        const uint64_t tiles = tile_count(kConfigs[cand.id], M, N);
        const uint64_t rounds = (tiles + kCUs - 1) / kCUs;
        const double cost = (double)rounds * cand.units / (rounds >= 2 ? cand.rate_many : cand.rate_one);
        if (first || cost < best_cost) {
            best = cand.id;
            best_cost = cost;
            first = false;
        }
    }
    return best;
}

// Argument checks shared by the entry points. Returns 0 or -position (sgemm numbering).
int check_args(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
               const float *C, int ldc)
{
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    if (reads_ab && A == nullptr) return -5;
    if (lda < (K > 1 ? K : 1)) return -6;
    if (reads_ab && B == nullptr) return -7;
    if (ldb < (N > 1 ? N : 1)) return -8;
    if (M > 0 && N > 0 && C == nullptr) return -10;
    if (ldc < (N > 1 ? N : 1)) return -11;
    return 0;
}

int run(int config, int M, int N, int K, float alpha, const float *A, int lda, int64_t sA,
        const float *B, int ldb, int64_t sB, float beta, float *C, int ldc, int64_t sC, int batch,
        hipStream_t stream)
{
    GemmArgs p;
    p.M = M; p.N = N; p.K = K;
    p.alpha = alpha; p.beta = beta;
    p.A = A; p.B = B; p.C = C;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.strideA = sA; p.strideB = sB; p.strideC = sC;

    if (K == 0 || alpha == 0.0f) {
        // C <- beta*C; A and B are not read.
        const int gx = (N + 255) / 256 < 64 ? (N + 255) / 256 : 64;
        const int gy = M < 1024 ? M : 1024;
        hipLaunchKernelGGL(sgemm_impl::sgemm_scale, dim3(gx, gy, batch), dim3(256, 1), 0, stream, p);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? 0 : (int)e;
    }
    const bool vec = vector_ok(N, K, A, lda, B, ldb, C, ldc) &&
                     (batch == 1 || (sA % 4 == 0 && sB % 4 == 0 && sC % 4 == 0));
    const int id = config >= 0 ? config : choose(M, N, vec);
    const Config &c = kConfigs[id];
    const uint64_t tiles = tile_count(c, M, N);
    if (c.kind == KIND_MFMA && tiles * (uint64_t)c.threads > 0xFFFFFFFFull)
        return SGEMM_ERROR_TOO_LARGE;
    const bool edge = (M % c.bm) != 0 || (N % c.bn) != 0 || (K % c.bk) != 0;
    const hipError_t e = c.launch(p, batch, vec, edge, stream);
    return e == hipSuccess ? 0 : (int)e;
}

}  // namespace

extern "C" {

int sgemm_ex(int config, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
             int ldb, float beta, float *C, int ldc, void *stream)
{
    if (config < -1 || config >= kNumConfigs)
        return SGEMM_ERROR_BAD_CONFIG;
    const int bad = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (bad != 0)
        return bad;
    if (M == 0 || N == 0)
        return SGEMM_SUCCESS;
    return run(config, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1,
               static_cast<hipStream_t>(stream));
}

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, void *stream)
{
    return sgemm_ex(-1, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_strided_batched(int M, int N, int K, float alpha, const float *A, int lda,
                          long long strideA, const float *B, int ldb, long long strideB, float beta,
                          float *C, int ldc, long long strideC, int batch, void *stream)
{
    // Positions: 1 M, 2 N, 3 K, 4 alpha, 5 A, 6 lda, 7 strideA, 8 B, 9 ldb, 10 strideB,
    // 11 beta, 12 C, 13 ldc, 14 strideC, 15 batch.
    static const int remap[12] = {0, -1, -2, -3, 0, -5, -6, -8, -9, 0, -12, -13};
    const int bad = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (bad != 0)
        return remap[-bad];
    if (strideA < 0) return -7;
    if (strideB < 0) return -10;
    if (batch < 0 || batch > 65535) return -15;
    if (batch > 1 && M > 0 && N > 0 && strideC < (long long)(M - 1) * ldc + N) return -14;
    if (M == 0 || N == 0 || batch == 0)
        return SGEMM_SUCCESS;
    return run(-1, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
               static_cast<hipStream_t>(stream));
}

int sgemm_config_count(void) { return kNumConfigs; }

const char *sgemm_config_name(int config)
{
    return (config >= 0 && config < kNumConfigs) ? kConfigs[config].name : nullptr;
}

int sgemm_select_config(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                        int ldb, const float *C, int ldc)
{
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.0f)
        return -1;
    return choose(M, N, vector_ok(N, K, A, lda, B, ldb, C, ldc));
}

int sgemm_launch_shape(int config, int M, int N, int K, int grid[3], int block[3])
{
    if (config < 0 || config >= kNumConfigs) return SGEMM_ERROR_BAD_CONFIG;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const Config &c = kConfigs[config];
    if (c.kind == KIND_TILE16) {
        grid[0] = (N + 15) / 16; grid[1] = (M + 15) / 16; grid[2] = 1;
        block[0] = 16; block[1] = 16; block[2] = 1;
        return 0;
    }
    const uint64_t tiles = tile_count(c, M, N);
    if (tiles * (uint64_t)c.threads > 0xFFFFFFFFull) return SGEMM_ERROR_TOO_LARGE;
    grid[0] = (int)tiles; grid[1] = 1; grid[2] = 1;
    block[0] = c.threads; block[1] = 1; block[2] = 1;
    return 0;
}

const char *sgemm_status_string(int status)
{
    switch (status) {
    case 0: return "success";
    case SGEMM_ERROR_TOO_LARGE: return "problem too large: the tile grid exceeds one launch";
    case SGEMM_ERROR_BAD_CONFIG: return "configuration id out of range";
    default: break;
    }
    if (status < 0 && status >= -16) {
        static const char *const msgs[17] = {
            "", "invalid argument 1", "invalid argument 2", "invalid argument 3", "invalid argument 4",
            "invalid argument 5", "invalid argument 6", "invalid argument 7", "invalid argument 8",
            "invalid argument 9", "invalid argument 10", "invalid argument 11", "invalid argument 12",
            "invalid argument 13", "invalid argument 14", "invalid argument 15", "invalid argument 16"};
        return msgs[-status];
    }
    if (status > 0)
        return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}

const char *sgemm_version(void) { return "tiled_fp32_gemm_02_amd 0.1 (gfx950)"; }

}  // extern "C"
