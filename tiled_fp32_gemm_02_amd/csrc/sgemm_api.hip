// C-ABI entry points of the fp32 GEMM library (declared in include/sgemm.h).
//
// Host work per call: validate the arguments (BLAS-style argument positions in the
// error code), take the quick returns (empty result; alpha == 0 or K == 0 leaves
// act(beta*C + bias)), choose a kernel configuration from the shape and alignment,
// and queue one kernel on the caller's stream. No allocation, copy or
// synchronisation. Stream-K launches use a workspace that the caller passes in.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "sgemm.h"
#include "sgemm_configs.inc"
#include "sgemm_aux_kernels.hpp"
#include "sgemm_launch.hpp"

using sgemm_impl::GemmArgs;

// Scratch of the allocation-free entry point (sgemm_general_noalloc): the stream-K workspace
// (tile counters, then partial-tile slots) as a file-scope device array, one copy per GPU,
// held until the process ends. Sized for both stream-K configurations on 256 compute units.
static __device__ __align__(256) unsigned char scratch[SGEMM_NOALLOC_SCRATCH_BYTES];

namespace {

using sgemm_impl::StreamK;

// ceil(a / b) for a >= 0, b >= 1, in 64 bits (a sum like a + b - 1 overflows int for a near 2^31).
uint64_t cdiv64(int a, int b) { return ((uint64_t)a + (uint64_t)b - 1) / (uint64_t)b; }

enum Kind { KIND_TILE16 = 0, KIND_MFMA = 1, KIND_SK = 2, KIND_VALU = 3 };

typedef hipError_t (*LaunchFn)(const GemmArgs &, int batch, bool ta, bool tb, bool vec, bool edge, bool dma_ok,
                               hipStream_t);
typedef hipError_t (*LaunchSkFn)(const GemmArgs &, const StreamK &, int grid, bool ta, bool tb, bool vec,
                                 bool edge, bool dma_ok, hipStream_t);

struct Config {
    const char *name;
    Kind kind;
    int bm, bn, bk;      // workgroup tile (tile16: 16 x 16 x 16)
    int threads;         // threads per workgroup
    bool dma;            // aligned operands are copied HBM -> LDS directly
    int group_m;         // band height of the tile order
    LaunchFn launch;     // data-parallel launch (KIND_TILE16, KIND_MFMA, KIND_VALU)
    LaunchSkFn launch_sk;    // stream-K launch (KIND_SK)
    int wgm, wgn, wgk;   // wave grid over the tile and wave groups along k (MFMA kinds)
    int pf;              // K-tiles whose loads run ahead of the one being multiplied
    int lds_bytes;       // static LDS per workgroup (aligned form)
    int unaligned_bk;    // K-tile of the form run for 4-byte aligned rows
    bool unaligned_dma;  // that form copies HBM -> LDS directly (else register-staged)
    int mb;              // block of the matrix instruction (32 or 16; 0 for the non-matrix kinds)
};

// LDS bytes and the unaligned form of an MFMA configuration, from the kernel's own
// constants (the same selection launch_mfma_op makes).
template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int MB>
struct MfmaFacts {
    static constexpr int NT = WGM * WGN * WGK * 64;
    static constexpr int LDS =
        4 * sgemm_impl::MfmaTile<BM, BN, BK, WGM, WGN, WGK, PF, DMA, false, false, true, false, MB>::SMEM;
    // Rows only 4-byte aligned: direct-copy configurations keep their tile and copies (the
    // K-tile holding the end of K in 4-byte words), register-staged ones their tile.
    static constexpr bool UDMA = DMA;
    static constexpr int UBK = BK;
};

// Stream-K workspace: per-tile counters at a fixed offset (so a call with more tiles
// never meets a previous call's partial sums there), then two partial-tile slots per
// workgroup.
constexpr int kSkMaxTiles = 16384;
constexpr size_t kSkCounterBytes = (size_t)kSkMaxTiles * sizeof(unsigned);

size_t sk_workspace_bytes(const Config &c, int cus)
{
    return kSkCounterBytes + (size_t)cus * 2 * (size_t)c.bm * (size_t)c.bn * sizeof(float);
}

// Compute units of the current device (one stream-K workgroup each), cached per device;
// 0 if the device cannot be queried.
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Row strides (floats) from which the direct-copy kernels' 32-bit in-tile offsets
// could overflow; such calls take the register-staged element-wise variant instead.
constexpr int kDmaMaxLd = 1 << 20;

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, int MB>
hipError_t launch_mfma(const GemmArgs &p, int batch, bool ta, bool tb, bool vec, bool edge, bool dma_ok,
                       hipStream_t s)
{
    if (!ta && !tb)
        return sgemm_impl::launch_mfma_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, false, false>(p, batch, vec,
                                                                                                     edge, dma_ok, s);
    if (!ta && tb)
        return sgemm_impl::launch_mfma_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, false, true>(p, batch, vec,
                                                                                                    edge, dma_ok, s);
    if (ta && !tb)
        return sgemm_impl::launch_mfma_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, true, false>(p, batch, vec,
                                                                                                    edge, dma_ok, s);
    return sgemm_impl::launch_mfma_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, true, true>(p, batch, vec, edge,
                                                                                               dma_ok, s);
}

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, int MB>
hipError_t launch_sk(const GemmArgs &p, const StreamK &sk, int grid, bool ta, bool tb, bool vec, bool edge,
                     bool dma_ok, hipStream_t s)
{
    if (!ta && !tb)
        return sgemm_impl::launch_mfma_sk_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, false, false>(
            p, sk, grid, vec, edge, dma_ok, s);
    if (!ta && tb)
        return sgemm_impl::launch_mfma_sk_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, false, true>(
            p, sk, grid, vec, edge, dma_ok, s);
    if (ta && !tb)
        return sgemm_impl::launch_mfma_sk_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, true, false>(
            p, sk, grid, vec, edge, dma_ok, s);
    return sgemm_impl::launch_mfma_sk_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, true, true>(
        p, sk, grid, vec, edge, dma_ok, s);
}

// The vector-ALU micro-tile kernel: one 256-thread workgroup per 128 x 128 tile.
hipError_t launch_valu(const GemmArgs &p, int batch, bool ta, bool tb, bool, bool, bool, hipStream_t s)
{
    constexpr int GROUP_M = 8;
    const unsigned tiles = (unsigned)(cdiv64(p.M, 128) * cdiv64(p.N, 128));   // checked by the caller
    const dim3 grid(tiles, 1, batch), block(256);
    if (!ta && !tb)
        hipLaunchKernelGGL((sgemm_impl::sgemm_valu<false, false>), grid, block, 0, s, p, GROUP_M);
    else if (!ta && tb)
        hipLaunchKernelGGL((sgemm_impl::sgemm_valu<false, true>), grid, block, 0, s, p, GROUP_M);
    else if (ta && !tb)
        hipLaunchKernelGGL((sgemm_impl::sgemm_valu<true, false>), grid, block, 0, s, p, GROUP_M);
    else
        hipLaunchKernelGGL((sgemm_impl::sgemm_valu<true, true>), grid, block, 0, s, p, GROUP_M);
    return hipGetLastError();
}

hipError_t launch_tile16(const GemmArgs &p, int batch, bool ta, bool tb, bool, bool, bool, hipStream_t s)
{
    const dim3 grid((unsigned)cdiv64(p.N, 16), (unsigned)cdiv64(p.M, 16), batch), block(16, 16);
    if (!ta && !tb)
        hipLaunchKernelGGL((sgemm_impl::sgemm_tile16<false, false>), grid, block, 0, s, p);
    else if (!ta && tb)
        hipLaunchKernelGGL((sgemm_impl::sgemm_tile16<false, true>), grid, block, 0, s, p);
    else if (ta && !tb)
        hipLaunchKernelGGL((sgemm_impl::sgemm_tile16<true, false>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((sgemm_impl::sgemm_tile16<true, true>), grid, block, 0, s, p);
    return hipGetLastError();
}

// Configuration table: id 0 is the 16x16 baseline kernel, then the MFMA configurations
// of sgemm_configs.inc in order, then its stream-K configurations, then the vector-ALU
// micro-tile kernel (tile 128 x 128 x 8, 8 x 8 outputs per thread). MFMA names encode the
// tile (BM x BN x BK), the wave grid (WGM x WGN), after "k" the wave groups along k, after
// "p" the K-tiles prefetched ahead (1 when absent), and a final "d" marks direct HBM -> LDS
// copies.
#define SGEMM_TABLE_ROW(name, BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB)                           \
    {name, KIND_MFMA, BM, BN, BK, WGM * WGN * WGK * 64, DMA != 0, GROUP_M,                                   \
     launch_mfma<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB>, nullptr, WGM, WGN, WGK, PF,                \
     MfmaFacts<BM, BN, BK, WGM, WGN, WGK, PF, DMA, MB>::LDS,                                                   \
     MfmaFacts<BM, BN, BK, WGM, WGN, WGK, PF, DMA, MB>::UBK, MfmaFacts<BM, BN, BK, WGM, WGN, WGK, PF, DMA, MB>::UDMA, \
     MB},
#define SGEMM_SK_TABLE_ROW(name, BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB)                        \
    {name, KIND_SK, BM, BN, BK, WGM * WGN * WGK * 64, DMA != 0, GROUP_M, nullptr,                            \
     launch_sk<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB>, WGM, WGN, WGK, PF,                          \
     MfmaFacts<BM, BN, BK, WGM, WGN, WGK, PF, DMA, MB>::LDS, BK, DMA != 0, MB},
// LDS of the two kernels outside the MFMA template: tile16 stages two 16 x 17 tiles; the
// vector-ALU kernel two k-major 8 x 132 tiles per stage, two stages.
const Config kConfigs[] = {
    {"tile16", KIND_TILE16, 16, 16, 16, 256, false, 1, launch_tile16, nullptr, 1, 1, 1, 0, 2 * 16 * 17 * 4, 16,
     false, 0},
    SGEMM_MFMA_CONFIGS(SGEMM_TABLE_ROW)
    SGEMM_SK_CONFIGS(SGEMM_SK_TABLE_ROW)
    {"valu_128x128x8_t8x8", KIND_VALU, 128, 128, 8, 256, false, 8, launch_valu, nullptr, 1, 1, 1, 1,
     2 * 2 * 8 * 132 * 4, 8, false, 0},
};
#undef SGEMM_TABLE_ROW
#undef SGEMM_SK_TABLE_ROW
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// 128-bit path: every operand 16-byte aligned, every row start 16-byte aligned, and
// each operand's contiguous extent a whole number of 4-float chunks (so a chunk is
// all in or all out): K for plain A, M for transposed A, N for plain B, K for
// transposed B, N for C.
bool vector_ok(int opA, int opB, int M, int N, int K, const float *A, int lda, const float *B, int ldb,
               const float *C, int ldc)
{
    return aligned16(A) && aligned16(B) && aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 && ldc % 4 == 0 &&
           (opA ? M : K) % 4 == 0 && (opB ? K : N) % 4 == 0 && N % 4 == 0;
}

uint64_t tile_count(const Config &c, int M, int N)
{
    return cdiv64(M, c.bm) * cdiv64(N, c.bn);
}

// Fringe columns of a data-parallel MFMA launch: when N mod BN = r is 1..kFringeCols, the
// whole tiles stop at column N - r and workgroups of their own, kFringeRows rows each, compute
// the last r columns (sgemm_mfma). Taken when the whole tiles still number at least
// kFringeMinTiles over the batch: a column of edge tiles then adds a round of tiles on
// some CUs, while in a smaller grid it runs beside the others. The fringe kernel indexes
// rows with 32-bit offsets, so it takes row strides under kDmaMaxLd only (ld_ok), and a
// grid too large for one launch with its fringe workgroups keeps the plain tiles. Returns
// r, or 0 for none.
constexpr uint64_t kFringeMinTiles = 256;
// Memory round trips of one fringe workgroup: its NT threads take 64 (NT / 64) U k per trip,
// U the k steps in flight per thread in fringe_columns (4 for up to 2 columns, 2 for 3-4, 1
// for 5-8; the kernel sets them to keep its registers low). Long K with many columns costs
// many trips: 999 x 999 x 3999 with 7 columns ran 7-36% slower on 16- and 32-wide tiles
// with the fringe (16 trips) than without, while one column at K = 777 (one trip) saved up to
// 39%. So the fringe is taken for at most kFringeMaxTrips.
// The fringe workgroups hold the kernel's LDS as its tiles do, so a CU runs as many of them
// at once as of the tiles: with 128 KiB tiles (256 x 256, 64 x 64 x 128) one, and then the
// ceil(M / 2) fringe workgroups of a tall product run in several rounds after the tiles (3072 x
// 3080 x 3072 on the 64 x 64 x 128 tile: six rounds, 516 us against 438 for 3072^3). The limit
// is on trips x rounds.
constexpr int kFringeMaxTrips = 3;
int fringe_trips(const Config &c, int K, int r)
{
    const int steps = r <= 2 ? 4 : r <= 4 ? 2 : 1;
    return (int)cdiv64(K, 64 * (c.threads / 64) * steps);
}
uint64_t fringe_rounds(const Config &c, int M, int batch)
{
    constexpr int kLdsPerCu = 160 * 1024, kWavesPerCu = 32, kCUs = 256;
    const int by_lds = c.lds_bytes > 0 ? kLdsPerCu / c.lds_bytes : kWavesPerCu;
    const int by_waves = kWavesPerCu / (c.threads / 64);
    int per_cu = by_lds < by_waves ? by_lds : by_waves;
    per_cu = per_cu > 0 ? per_cu : 1;
    const uint64_t slots = (uint64_t)kCUs * per_cu;
    return (cdiv64(M, sgemm_impl::kFringeRows) * (uint64_t)batch + slots - 1) / slots;
}
int fringe_cols(const Config &c, int M, int N, int K, int batch, bool ld_ok = true)
{
    if (c.kind != KIND_MFMA || N < c.bn || !ld_ok)
        return 0;
    const int r = N % c.bn;
    if (r == 0 || r > sgemm_impl::kFringeCols)
        return 0;
    const uint64_t whole = cdiv64(M, c.bm) * (uint64_t)(N / c.bn);
    if (whole * (uint64_t)batch < kFringeMinTiles)
        return 0;
    if ((uint64_t)fringe_trips(c, K, r) * fringe_rounds(c, M, batch) > (uint64_t)kFringeMaxTrips)
        return 0;
    // ceil(M / kFringeRows) more workgroups: a grid that would then pass one launch's
    // 2^32 threads keeps its plain column of edge tiles instead
    const uint64_t wgs = whole + cdiv64(M, sgemm_impl::kFringeRows);
    return wgs * (uint64_t)c.threads <= 0xFFFFFFFFull ? r : 0;
}

// Whole tiles of a launch with `fringe` fringe columns, and all its workgroups (per batch entry).
uint64_t main_tiles(const Config &c, int M, int N, int fringe)
{
    return fringe > 0 ? cdiv64(M, c.bm) * (uint64_t)((N - fringe) / c.bn) : tile_count(c, M, N);
}
uint64_t grid_count(const Config &c, int M, int N, int fringe)
{
    return main_tiles(c, M, N, fringe) + (fringe > 0 ? cdiv64(M, sgemm_impl::kFringeRows) : 0);
}

// The stream-K kernel splits work with 32-bit arithmetic: (CUs + 1) * work < 2^31.
// Stream-K split of `tiles` tiles of `iters` K-tiles over `cus` CUs. Direct-copy
// configurations (`whole` true) run whole rounds of tiles, one per CU each, except the last
// round, as plain tiles (the first dp tiles), and share the last round's tiles; register-
// staged ones share every tile (dp = 0): their stream-K kernels hold more than 128 registers,
// so only one workgroup fits a CU and whole-tile rounds beside the shared one would not
// overlap. The shared steps go to one workgroup per CU, or one per step when there are
// fewer, so every range is non-empty. dp is a whole number of XCD rounds (8), as the
// kernel's workgroup order needs. Returns the grid.
int sk_split(int tiles, int iters, int cus, bool whole, int &dp)
{
    dp = whole && tiles > cus ? (tiles - 1) / cus * cus : 0;
    dp -= dp % 8;
    const int shared = (tiles - dp) * iters;
    return dp + (shared < cus ? shared : cus);
}

bool sk_work_fits(const Config &c, int M, int N, int K, int cus)
{
    const uint64_t tiles = tile_count(c, M, N);
    const uint64_t work = tiles * cdiv64(K, c.bk);
    return tiles <= (uint64_t)kSkMaxTiles && work * (uint64_t)(cus + 1) < (1ull << 31);
}

// Auto-selection by a small cost model of the kernel time, measured on MI355X.
//
// A candidate's time is the largest of three bounds:
//  - compute: the tiles spread over the CUs take L = ceil(tiles / CUs) rounds on the
//    busiest CU, so the time is a fixed cost (launch, first loads, last epilogue), a cost
//    per round (a tile's first loads and epilogue, which short K loops do not hide) and L
//    tiles of work (one unit is a 64 x 64 tile, 2 * 64 * 64 * K flop) at the CU's measured
//    speed, given as microseconds per MFLOP with one workgroup resident (L = 1) or
//    several (L >= 2). Stream-K candidates (only with a large enough workspace) give
//    every CU the same share, tiles * units / CUs, at the one- or several-workgroup speed
//    (several when whole-tile rounds run beside the shared one), plus a fixed cost and a
//    cost per round.
//  - HBM: each operand's compulsory bytes (A and B read, C written) at a bandwidth that
//    depends on the contiguous bytes per row a tile reads (BK floats of A, BN of B and C):
//    5.7 TB/s for 512-byte rows, falling as (bytes / 512)^0.19 for shorter ones (measured
//    from 3.8 TB/s at 64 bytes to 5.7 TB/s on products that stream one operand).
//  - L2: the tiles' operand panels, 4 M N K (1 / BM + 1 / BN) bytes, at the highest rate
//    any swept configuration reached on them (20 TB/s for 16-byte aligned rows, 14 TB/s
//    for 4-byte aligned ones). Small tiles re-read panels many times, and on long-K
//    products such as 1024 x 768 x 3072 that, not the matrix cores, sets their time.
struct Candidate {
    const char *name;   // configuration name in the table
    double fixed_us;    // time that does not scale with the work
    double round_us;    // time per round of tiles on a CU beyond its work
    double us_one;      // microseconds per MFLOP of a CU's work with one workgroup resident
    double us_many;     // the same with two or more
};

// Non-negative least-squares fits (relative error) of the compute bound, per operand
// alignment, over the shapes of one sweep where neither memory bound was within 75% of the
// measured time. Aligned: 36 single products (256^3 ... 6144^3, 3000^3, rectangles, the
// GPT-2-small linear layers, long-K and skinny products down to 16 rows or columns) and 10
// batched ones at half weight (attention's 12-head products 1024 x 1024 x 64 and
// 1024 x 64 x 1024, the first with K from 16 to 256, and 48 or 3 heads of other sizes),
// whose short K loops set the per-round costs. Unaligned (rows only 4-byte aligned): 24
// odd-sized shapes (255^3 ... 6143^3, 2999^3, 511 x 4095 x 4095, 1000 x 1537 x 777, the
// GPT-2 layers one short in each dimension, long-K and skinny ones). Candidates were chosen
// by dropping, one at a time, those whose removal improved the picks, scored both for
// callers with a stream-K workspace and without one. Aligned, the picks average within
// 1.4% of the fastest of all those swept; the benchmark shapes get the fastest (the GPT-2
// QKV layer and 1536^3 on the 16x16-block stream-K tile when a workspace is passed) except
// the attention values product (7%); the worst misses are 16384 x 16 x 16384 (19%), 768^3
// (13%) and 16 x 16384 x 16384 (8%). Unaligned, within 0.6% on average and 5.7% at worst,
// the ragged 1000 x 1537 x 777 at 2.4% (33.5 against 32.7 us for the 64 x 128 tile).
const Candidate kCandidates[] = {
    {"mfma_128x128x32_w2x2k2d", 0.00, 5.53, 1.8246, 1.7719},
    {"mfma_256x128x32_w4x2d", 0.00, 0.00, 1.9088, 3.3975},
    {"mfma_256x256x32_w2x4d", 0.00, 10.68, 1.7024, 1.7316}, // one workgroup per CU (4096^3)
    {"mfma_32x128x64_w1x4k2d", 2.09, 1.92, 2.2306, 1.9510},
    {"mfma_32x32x64_w1x1k4d", 2.02, 0.84, 4.6692, 2.1984}, // GPT-2 MLP-down
    {"mfma_32x64x64_w1x2k2d", 2.66, 1.11, 2.5009, 2.0088},
    {"mfma_32x96x64_w1x1k4d", 3.32, 2.26, 2.5438, 2.1241},
    {"mfma_64x128x32_w2x2k2d", 0.70, 2.33, 2.0154, 1.7883},
    {"mfma_64x64x32_w2x2k2d", 0.00, 2.00, 2.7466, 1.9709},
    {"mfma_64x64x64_w2x2k4d", 0.20, 4.07, 2.1338, 1.9515},
    {"mfma16_128x64x32_w8x1k1d", 0.45, 1.61, 2.0761, 1.8242},
    {"mfma16_16x16x128_w1x1k4d", 2.15, 0.50, 16.3796, 2.7659},
    {"mfma16_16x16x128_w1x1k4p2d", 2.66, 0.49, 9.5499, 3.4119},
    {"mfma16_16x16x256_w1x1k4d", 1.99, 0.87, 10.9830, 3.5898}, // 256^3
    {"mfma16_16x64x128_w1x1k4d", 2.34, 0.70, 3.5422, 2.4972},
    {"mfma16_32x128x64_w2x2k2d", 1.57, 1.35, 2.2657, 1.9571},
    {"mfma16_32x32x128_w2x2k2d", 1.99, 0.99, 2.8169, 2.2152},
    {"mfma16_32x32x64_w2x2k1d", 2.11, 0.40, 4.1882, 2.3430}, // attention values
    {"mfma16_32x64x128_w2x1k4d", 0.99, 2.40, 2.0417, 2.0110},
    {"mfma16_32x96x128_w2x2k4d", 0.91, 3.37, 2.3607, 2.2939},
    {"mfma16_32x96x64_w2x2k2d", 2.09, 1.14, 2.8095, 2.2418}, // GPT-2 QKV without a workspace
    {"mfma16_64x128x32_w4x2k1d", 0.56, 1.63, 1.9927, 1.7666}, // attention scores
    {"mfma16_64x16x64_w4x1k1d", 2.09, 0.27, 4.5657, 2.7117},
    {"mfma16_64x64x128_w4x1k4d", 0.00, 4.26, 1.9058, 1.7591},
    {"mfma16_64x64x32_w4x1k1d", 0.08, 0.86, 2.7331, 1.8368}, // GPT-2 MLP-up
    {"mfma16_64x64x64_w2x2k2d", 1.26, 1.35, 2.0657, 1.8103},
    {"mfma16_64x64x64_w4x1k2d", 1.28, 1.32, 2.0562, 1.8045}, // 1024^3
    {"mfma16_64x96x64_w4x2k1d", 2.02, 1.26, 2.4321, 2.1043},
};
const Candidate kUnalignedCandidates[] = {
    {"mfma_256x256x32_w2x4d", 14.80, 0.00, 1.7815, 1.8531},
    {"mfma_256x256x16_w2x4p2d", 14.57, 0.00, 1.7493, 1.7959},
    {"mfma_128x128x32_w2x2k2d", 9.76, 0.00, 1.8352, 1.8036},
    {"mfma_64x128x32_w2x2k2d", 4.27, 2.30, 1.9893, 1.7655},
    {"mfma_64x64x32_w2x2k2d", 1.90, 3.53, 2.7001, 1.8506},
    {"mfma_32x128x64_w1x4k2d", 2.71, 4.98, 2.2361, 1.8618},
    {"mfma_32x64x64_w1x2k2d", 5.17, 2.49, 2.7631, 1.9155},
    {"mfma16_128x64x32_w8x1k1d", 2.61, 4.06, 2.1476, 1.8057},
    {"mfma16_64x128x32_w4x2k1d", 0.92, 5.31, 2.1907, 1.7932},
    {"mfma16_64x64x64_w4x1k2d", 1.24, 4.14, 2.1442, 1.8001},
    {"mfma16_64x64x64_w2x2k2d", 1.05, 3.96, 2.2426, 1.8103},
    {"mfma16_64x64x32_w4x1k1d", 2.57, 2.03, 2.7560, 1.9233},
    {"mfma16_64x16x64_w4x1k1d", 3.94, 0.00, 5.8194, 3.2452},
    {"mfma16_32x128x64_w2x2k2d", 0.20, 4.99, 2.2661, 1.8105},
    {"mfma16_32x64x128_w2x1k4d", 0.88, 5.66, 2.3716, 2.3479},
    {"mfma16_32x64x64_w2x1k2d", 4.03, 1.07, 3.1605, 2.1120}, // 1000 x 1537 x 777 (a fringe column)
    {"mfma16_32x32x128_w2x2k2d", 3.09, 2.02, 3.5613, 2.4795},
    {"mfma16_32x32x64_w2x2k1d", 3.62, 0.93, 4.9384, 2.4736},
    {"mfma16_16x64x128_w1x1k4d", 5.14, 2.17, 4.0984, 3.0357},
    {"mfma16_16x16x256_w1x1k4d", 2.71, 2.32, 12.8062, 4.1227},
    {"mfma16_16x16x128_w1x1k4p2d", 4.83, 1.18, 3.0145, 4.2636},
    {"mfma16_16x16x128_w1x1k4d", 2.96, 0.69, 14.9652, 4.2246},
    {"mfma_32x96x64_w1x1k4d", 3.03, 5.42, 2.6653, 1.9967},
    {"mfma16_32x96x32_w2x2k1d", 4.79, 0.55, 3.7010, 2.3138}, // GPT-2 QKV one short
    {"mfma16_32x96x64_w2x2k2d", 1.94, 3.24, 2.7101, 2.1268},
    {"mfma16_64x96x64_w4x2k1d", 2.12, 4.06, 2.3739, 2.0297},
    {"mfma16_32x96x128_w2x2k4d", 2.14, 6.34, 2.1533, 2.2237}, // GPT-2 MLP-down one short
    {"mfma16_64x64x128_w4x1k4d", 1.60, 6.32, 1.9030, 1.9336}, // long K (999 x 999 x 3999)
};
// Strided-batched products (batch > 1, aligned or not) take their own short list,
// fitted on batched shapes only (attention-like products: 12 to 48 heads of 1024 x 1024 x 16..256
// and of 1024 x 64 x 1024..4096, 3 x 2048^2 x 64 and 4096^2 x 64, 16 x 256^3 and 16 x 128^2 x 64,
// and the shapes with a 64-wide output): the single-product list, whose larger tiles were never
// swept on batched shapes, sent 12 x 1024^2 x 16 and x 32 to the 256 x 128 tile (30-36% behind).
// With this list the picks average within 2.1% of the fastest measured on 34 batched shapes.
// Batches of a few large products (2 x 1024 x 2304 x 768) took the 32 x 32 tile, 15-24%
// behind the 64 x 96 one; that tile, fitted alone with the other three unchanged, joined last.
// Operands only 4-byte aligned run the same tiles with their unaligned direct copies: on
// 12-head attention shapes with K or N of 63, 65, 127 or 17 and on 16 x 255^3 these tiles
// ran 5-47% ahead of the 128 x 128 tile the unaligned single-product list picked there; the
// picks came within 6% of the fastest measured but for 16 x 255^3 (the 16 x 64 tile, 12.6 us
// against 10.6 us for the 64 x 64 tile of the single-product list).
const Candidate kBatchedCandidates[] = {
    {"mfma16_64x128x32_w4x2k1d", 1.61, 1.51, 2.0773, 1.7591}, // attention scores
    {"mfma16_16x64x64_w1x1k4d", 3.07, 0.63, 8.4280, 2.1437},  // attention values
    {"mfma16_32x32x64_w2x2k1d", 4.45, 0.48, 0.0000, 2.0692},
    {"mfma16_64x96x64_w4x2k1d", 7.13, 0.67, 2.1684, 2.0067},  // a few large products (2 x QKV)
};
const Candidate kSkCandidates[] = {
    {"sk16_32x64x64_w2x1k2d", 6.48, 0.00, 3.8051, 2.2519},
    {"sk16_64x64x32_w4x1k1d", 7.97, 0.00, 3.4711, 1.9340}, // GPT-2 QKV, 1536^3, 2560^3
    {"sk_128x128x32_w2x2k2p2", 0.00, 20.97, 1.8670, 0.0000},
    {"sk_64x128x32_w2x2k2p2", 0.00, 12.80, 2.0335, 0.0000}, // long K, few tiles
};
const Candidate kSkUnalignedCandidates[] = {
    {"sk_64x128x32_w2x2k2d", 15.23, 0.00, 2.0518, 1.7418}, // 1535^3, 2999^3
    {"sk16_64x64x32_w4x1k1d", 11.80, 0.00, 2.7649, 1.9380},
    {"sk16_32x64x64_w2x1k2d", 9.13, 1.23, 2.9773, 2.1127},
};
constexpr int kNumCandidates = sizeof(kCandidates) / sizeof(kCandidates[0]);
constexpr int kNumUnalignedCandidates = sizeof(kUnalignedCandidates) / sizeof(kUnalignedCandidates[0]);
constexpr int kNumSkCandidates = sizeof(kSkCandidates) / sizeof(kSkCandidates[0]);
constexpr int kNumBatchedCandidates = sizeof(kBatchedCandidates) / sizeof(kBatchedCandidates[0]);
constexpr int kNumSkUnalignedCandidates = sizeof(kSkUnalignedCandidates) / sizeof(kSkUnalignedCandidates[0]);
// A stream-K candidate is taken only when its modelled time, 3% longer, still beats the
// data-parallel one: its shared tiles are the part of the model with the widest spread.
constexpr double kSkMargin = 1.03;
// Modelled time of a launch's fringe workgroups beyond its tiles (us): fixed, and per memory
// round trip of one fringe workgroup and round of fringe workgroups.
constexpr double kFringeTripUs = 1.0, kFringeFixedUs = 1.0;
constexpr double kHbmBytesPerUs = 5.7e6;          // 5.7 TB/s for rows of 512 contiguous bytes
constexpr double kHbmRowExponent = 0.19;
constexpr double kL2BytesPerUs = 20.0e6;          // tile-fill bytes, 16-byte aligned rows
constexpr double kL2BytesPerUsUnaligned = 16.8e6;  // and 4-byte aligned rows

int find_config(const char *name)
{
    for (int i = 0; i < kNumConfigs; ++i) {
        const char *a = kConfigs[i].name, *b = name;
        while (*a && *a == *b) { ++a; ++b; }
        if (*a == *b)
            return i;
    }
    return -1;
}

// Table ids of the candidates, looked up once.
struct CandidateIds {
    int id[kNumCandidates], un[kNumUnalignedCandidates], sk[kNumSkCandidates], sku[kNumSkUnalignedCandidates];
    int bt[kNumBatchedCandidates];
    CandidateIds()
    {
        for (int i = 0; i < kNumBatchedCandidates; ++i) bt[i] = find_config(kBatchedCandidates[i].name);
        for (int i = 0; i < kNumCandidates; ++i) id[i] = find_config(kCandidates[i].name);
        for (int i = 0; i < kNumUnalignedCandidates; ++i) un[i] = find_config(kUnalignedCandidates[i].name);
        for (int i = 0; i < kNumSkCandidates; ++i) sk[i] = find_config(kSkCandidates[i].name);
        for (int i = 0; i < kNumSkUnalignedCandidates; ++i) sku[i] = find_config(kSkUnalignedCandidates[i].name);
    }
};

// The two memory bounds of configuration c on `batch` products of M x N x K, in us.
double memory_us(const Config &c, int M, int N, int K, int batch, bool vec)
{
    auto bw = [](double row_bytes) {
        const double r = row_bytes < 512.0 ? row_bytes / 512.0 : 1.0;
        return kHbmBytesPerUs * std::pow(r, kHbmRowExponent);
    };
    const double m = M, n = N, k = K, b = batch;
    const double hbm = b * (4.0 * m * k / bw(4.0 * c.bk) + 4.0 * k * n / bw(4.0 * c.bn) + 4.0 * m * n / bw(4.0 * c.bn));
    const double l2 = b * 4.0 * m * n * k * (1.0 / c.bm + 1.0 / c.bn) / (vec ? kL2BytesPerUs : kL2BytesPerUsUnaligned);
    return hbm > l2 ? hbm : l2;
}

// The configuration with the least modelled time. Stream-K candidates are considered
// only for one product (batch 1), when `ws_bytes` holds their workspace for `cus` compute
// units (cus > 0); for operands only 4-byte aligned, only direct-copy ones.
int choose_model(int M, int N, int K, bool vec, size_t ws_bytes, int cus, int batch)
{
    static const CandidateIds ids;
    const bool batched = batch > 1;
    const Candidate *table = batched ? kBatchedCandidates : vec ? kCandidates : kUnalignedCandidates;
    const int *table_ids = batched ? ids.bt : vec ? ids.id : ids.un;
    const int table_len = batched ? kNumBatchedCandidates : vec ? kNumCandidates : kNumUnalignedCandidates;
    const uint64_t kCUs = cus > 0 ? (uint64_t)cus : 256;
    const double unit_mflop = 2.0 * 64 * 64 * (double)K * 1e-6;    // one 64x64 tile, MFLOP
    int best = -1;
    double best_us = 0.0;
    for (int i = 0; i < table_len; ++i) {
        const Candidate &cand = table[i];
        if (table_ids[i] < 0)
            continue;
        const Config &c = kConfigs[table_ids[i]];
        const int fringe = fringe_cols(c, M, N, K, batch);
        const uint64_t tiles = main_tiles(c, M, N, fringe) * (uint64_t)batch;
        const uint64_t rounds = (tiles + kCUs - 1) / kCUs;
        const double units = (double)c.bm * c.bn / 4096.0;
        double us = cand.fixed_us + (double)rounds * cand.round_us +
                    (double)rounds * units * unit_mflop * (rounds >= 2 ? cand.us_many : cand.us_one) +
                    (fringe > 0 ? kFringeFixedUs + kFringeTripUs * fringe_trips(c, K, fringe) *
                                      (double)fringe_rounds(c, M, batch) : 0.0);
        const double mem = memory_us(c, M, N, K, batch, vec);
        us = us > mem ? us : mem;
        if (best < 0 || us < best_us) {
            best = table_ids[i];
            best_us = us;
        }
    }
    const Candidate *sk_table = vec ? kSkCandidates : kSkUnalignedCandidates;
    const int *sk_ids = vec ? ids.sk : ids.sku;
    const int sk_len = vec ? kNumSkCandidates : kNumSkUnalignedCandidates;
    for (int i = 0; cus > 0 && batch == 1 && i < sk_len; ++i) {
        const Candidate &cand = sk_table[i];
        if (sk_ids[i] < 0)
            continue;
        const Config &c = kConfigs[sk_ids[i]];
        const uint64_t tiles = tile_count(c, M, N);
        if (!sk_work_fits(c, M, N, K, cus) || ws_bytes < sk_workspace_bytes(c, cus))
            continue;
        // whole-tile rounds (dp / CUs of them) and the shared last round, with the CU's
        // work spread evenly; one workgroup per CU when every tile is shared (dp = 0)
        int dp = 0;
        sk_split((int)tiles, (int)cdiv64(K, c.bk), cus, c.dma, dp);
        const double units = (double)c.bm * c.bn / 4096.0;
        double us = cand.fixed_us + ((double)dp / (double)kCUs + 1.0) * cand.round_us +
                    (double)tiles * units / (double)kCUs * unit_mflop * (dp == 0 ? cand.us_one : cand.us_many);
        const double mem = memory_us(c, M, N, K, 1, vec);
        us = us > mem ? us : mem;
        if (us * kSkMargin < best_us) {
            best = sk_ids[i];
            best_us = us * kSkMargin;
        }
    }
    return best;
}

// The same choice with a small per-thread memo of recent queries: the pick depends only on
// these arguments, and the model costs about 2 us of host time per call, as much as a small
// product's kernel. Calls that repeat a shape, as training and serving loops do, skip it.
int choose(int M, int N, int K, bool vec, size_t ws_bytes = 0, int cus = 0, int batch = 1)
{
    struct Query {
        int M, N, K, cus, batch;
        size_t ws_bytes;
        bool vec;
        int id;
    };
    constexpr int kMemo = 8;
    thread_local Query memo[kMemo];
    thread_local int used = 0, next = 0;
    for (int i = 0; i < used; ++i) {
        const Query &q = memo[i];
        if (q.M == M && q.N == N && q.K == K && q.cus == cus && q.batch == batch && q.ws_bytes == ws_bytes &&
            q.vec == vec)
            return q.id;
    }
    const int id = choose_model(M, N, K, vec, ws_bytes, cus, batch);
    memo[next] = Query{M, N, K, cus, batch, ws_bytes, vec, id};
    next = (next + 1) % kMemo;
    used = used < kMemo ? used + 1 : kMemo;
    return id;
}

// Arguments that can be invalid, independent of any entry point's numbering.
enum Arg { ARG_OK = 0, ARG_OPA, ARG_OPB, ARG_M, ARG_N, ARG_K, ARG_A, ARG_LDA, ARG_B, ARG_LDB, ARG_C, ARG_LDC,
           ARG_ACT };

// The first invalid argument, in declaration order, or ARG_OK.
Arg check_args(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
               int ldb, const float *C, int ldc, int act)
{
    if (opA != SGEMM_OP_N && opA != SGEMM_OP_T) return ARG_OPA;
    if (opB != SGEMM_OP_N && opB != SGEMM_OP_T) return ARG_OPB;
    if (M < 0) return ARG_M;
    if (N < 0) return ARG_N;
    if (K < 0) return ARG_K;
    const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    if (reads_ab && A == nullptr) return ARG_A;
    const int a_cols = opA ? M : K;     // the contiguous extent of A as stored
    if (lda < (a_cols > 1 ? a_cols : 1)) return ARG_LDA;
    if (reads_ab && B == nullptr) return ARG_B;
    const int b_cols = opB ? K : N;
    if (ldb < (b_cols > 1 ? b_cols : 1)) return ARG_LDB;
    if (M > 0 && N > 0 && C == nullptr) return ARG_C;
    if (ldc < (N > 1 ? N : 1)) return ARG_LDC;
    if (act != SGEMM_ACT_NONE && act != SGEMM_ACT_GELU_TANH) return ARG_ACT;
    return ARG_OK;
}

// Positions (1-based) of each Arg in the entry points' signatures; 0 = not an argument.
//                       OK opA opB M  N  K  A  lda B  ldb C   ldc act
const int kPosPlain[] = {0, 0, 0, 1, 2, 3, 5, 6, 7, 8, 10, 11, 0};     // sgemm, sgemm_ex
const int kPosOp[] = {0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 12, 13, 0};       // sgemm_op
const int kPosFused[] = {0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 12, 13, 15};   // sgemm_bias_act, sgemm_general
const int kPosBatched[] = {0, 0, 0, 1, 2, 3, 5, 6, 8, 9, 12, 13, 0};   // sgemm_strided_batched
const int kPosBatchedOp[] = {0, 1, 2, 3, 4, 5, 7, 8, 10, 11, 14, 15, 18};  // sgemm_strided_batched_op/general

// Batched calls: strides and count valid, and the batches' C windows disjoint. Windows are
// disjoint when they are stacked (each starts past the previous one's last entry) or side by
// side inside the rows of one matrix (each N wide, all of them within ldc), as when attention
// heads write their columns of one output. Returns 0, or the position of the bad argument
// given the positions of strideA, strideB, strideC and batch.
int check_batch(int M, int N, int ldc, long long sA, long long sB, long long sC, int batch, int pA, int pB,
                int pC, int pBatch)
{
    if (sA < 0) return pA;
    if (sB < 0) return pB;
    if (sC < 0) return pC;
    if (batch < 0 || batch > 65535) return pBatch;
    // The last batch's offset (batch - 1) * stride stays far inside 64-bit arithmetic.
    const long long kMaxOffset = 1LL << 60;
    if (batch > 1) {
        if (sA > kMaxOffset / (batch - 1)) return pA;
        if (sB > kMaxOffset / (batch - 1)) return pB;
        if (sC > kMaxOffset / (batch - 1)) return pC;
    }
    if (batch > 1 && M > 0 && N > 0) {
        const bool stacked = sC >= (long long)(M - 1) * ldc + N;
        const bool side_by_side = sC >= N && (long long)(batch - 1) * sC + N <= ldc;
        if (!stacked && !side_by_side) return pC;
    }
    return 0;
}

int run(int config, int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda, int64_t sA,
        const float *B, int ldb, int64_t sB, float beta, float *C, int ldc, int64_t sC, const float *bias,
        int act, int batch, void *ws, size_t ws_bytes, hipStream_t stream)
{
    GemmArgs p;
    p.M = M; p.N = N; p.K = K;
    p.alpha = alpha; p.beta = beta;
    p.A = A; p.B = B; p.C = C;
    p.bias = bias; p.act = act; p.fringe = 0;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.strideA = sA; p.strideB = sB; p.strideC = sC;

    if (K == 0 || alpha == 0.0f) {
        // C <- act(beta*C + bias); A and B are not read.
        sgemm_impl::StridedArgs q;
        static_cast<GemmArgs &>(q) = p;
        q.incA = q.incB = q.incC = 1;
        const int gx = cdiv64(N, 256) < 64 ? (int)cdiv64(N, 256) : 64;
        const int gy = M < 1024 ? M : 1024;
        hipLaunchKernelGGL(sgemm_impl::sgemm_scale, dim3(gx, gy, batch), dim3(256, 1), 0, stream, q);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? 0 : (int)e;
    }
    const bool vec = vector_ok(opA, opB, M, N, K, A, lda, B, ldb, C, ldc) &&
                     (batch == 1 || (sA % 4 == 0 && sB % 4 == 0 && sC % 4 == 0));
    const int cus = (ws != nullptr && batch == 1) ? device_cus() : 0;
    const int id = config >= 0 ? config : choose(M, N, K, vec, ws_bytes, cus, batch);
    const Config &c = kConfigs[id];
    const int fringe = fringe_cols(c, M, N, K, batch, lda < kDmaMaxLd && ldb < kDmaMaxLd);
    const uint64_t tiles = tile_count(c, M, N);
    if ((c.kind == KIND_MFMA || c.kind == KIND_VALU) && grid_count(c, M, N, fringe) * (uint64_t)c.threads > 0xFFFFFFFFull)
        return SGEMM_ERROR_TOO_LARGE;
    p.fringe = fringe;
    const bool edge = (M % c.bm) != 0 || ((N - fringe) % c.bn) != 0 || (K % c.bk) != 0;
    // Direct copies address a tile with 32-bit offsets, so long rows take the register-staged
    // kernels; so do row strides under 4 floats, where a 16-byte copy of a row's last chunk
    // could pass more than the next row.
    const bool dma_ok = lda < kDmaMaxLd && ldb < kDmaMaxLd && lda >= 4 && ldb >= 4;
    if (c.kind == KIND_SK) {
        if (batch != 1 || cus <= 0 || ws_bytes < sk_workspace_bytes(c, cus))
            return SGEMM_ERROR_WORKSPACE;
        if (!sk_work_fits(c, M, N, K, cus))
            return SGEMM_ERROR_TOO_LARGE;
        StreamK sk;
        sk.counters = static_cast<unsigned *>(ws);
        sk.partials = reinterpret_cast<float *>(static_cast<char *>(ws) + kSkCounterBytes);
        sk.tiles_m = (int)cdiv64(M, c.bm);
        sk.tiles_n = (int)cdiv64(N, c.bn);
        sk.iters = (int)cdiv64(K, c.bk);
        sk.group_m = c.group_m;
        sk.work = (int)tiles * sk.iters;
        const int grid = sk_split((int)tiles, sk.iters, cus, c.dma, sk.dp);
        const hipError_t e = c.launch_sk(p, sk, grid, opA != 0, opB != 0, vec, edge, dma_ok, stream);
        return e == hipSuccess ? 0 : (int)e;
    }
    const hipError_t e = c.launch(p, batch, opA != 0, opB != 0, vec, edge, dma_ok, stream);
    return e == hipSuccess ? 0 : (int)e;
}

int general(const int *pos, int config, int opA, int opB, int M, int N, int K, float alpha, const float *A,
            int lda, const float *B, int ldb, float beta, float *C, int ldc, const float *bias, int act,
            void *stream, void *ws = nullptr, size_t ws_bytes = 0)
{
    if (config < -1 || config >= kNumConfigs)
        return SGEMM_ERROR_BAD_CONFIG;
    const Arg bad = check_args(opA, opB, M, N, K, alpha, A, lda, B, ldb, C, ldc, act);
    if (bad != ARG_OK)
        return -pos[bad];
    if (M == 0 || N == 0)
        return SGEMM_SUCCESS;
    return run(config, opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, bias, act, 1, ws,
               ws_bytes, static_cast<hipStream_t>(stream));
}

// General-stride operands: op(A)(i,k) = A[i*rsA + k*csA], B(k,j) = B[k*rsB + j*csB],
// C(i,j) = C[i*rsC + j*csC]. Layouts the stored-matrix forms already cover (a unit stride in
// one dimension, the other at least the extent it spans) run through them with the auto
// choice; a column-major C without bias runs as the transposed product C^T = B^T A^T; every
// other layout runs the general-stride tile kernel.

// An operand of `rows` x `cols` with row stride rs and column stride cs as a stored-matrix
// form: op SGEMM_OP_N with ld = rs, or SGEMM_OP_T with ld = cs. False if neither fits.
bool as_stored(int rows, int cols, long long rs, long long cs, int &op, int &ld)
{
    const long long kMaxLd = 0x7fffffffLL;
    if (cols <= 1) {                            // one column: element i at i*rs
        op = SGEMM_OP_N;
        if (rows <= 1) { ld = 1; return true; }
        if (rs < 1 || rs > kMaxLd) return false;
        ld = (int)rs;
        return true;
    }
    if (rows <= 1) {                            // one row: element j at j*cs
        if (cs == 1) { op = SGEMM_OP_N; ld = cols; return true; }
        if (cs < 1 || cs > kMaxLd) return false;
        op = SGEMM_OP_T; ld = (int)cs;         // stored as a cols x 1 column of stride cs
        return true;
    }
    if (cs == 1 && rs >= cols && rs <= kMaxLd) { op = SGEMM_OP_N; ld = (int)rs; return true; }
    if (rs == 1 && cs >= rows && cs <= kMaxLd) { op = SGEMM_OP_T; ld = (int)cs; return true; }
    return false;
}

hipError_t launch_strided(const sgemm_impl::StridedArgs &p, hipStream_t s)
{
    // The register-staged 64 x 64 tile of two wave groups (mfma_64x64x32_w2x2k2's shape).
    constexpr int BM = 64, BN = 64, BK = 32, WGM = 2, WGN = 2, WGK = 2, MB = 32, GROUP_M = 8;
    const unsigned tiles = (((unsigned)p.M + BM - 1) / BM) * (((unsigned)p.N + BN - 1) / BN);
    hipLaunchKernelGGL((sgemm_impl::sgemm_mfma_strided<BM, BN, BK, WGM, WGN, WGK, MB>), dim3(tiles),
                       dim3(WGM * WGN * WGK * 64), 0, s, p, GROUP_M);
    return hipGetLastError();
}

int strided(int M, int N, int K, float alpha, const float *A, long long rsA, long long csA, const float *B,
            long long rsB, long long csB, float beta, float *C, long long rsC, long long csC, const float *bias,
            int act, hipStream_t stream)
{
    if (M == 0 || N == 0)
        return SGEMM_SUCCESS;
    if (K == 0 || alpha == 0.0f || (csC == 1 || N == 1)) {
        int opA = SGEMM_OP_N, opB = SGEMM_OP_N, lda = 1, ldb = 1, ldc = 1;
        const bool quick = K == 0 || alpha == 0.0f;
        const bool c_rows = (csC == 1 || N == 1) && (M == 1 || (rsC >= N && rsC <= 0x7fffffffLL));
        if (c_rows)
            ldc = M == 1 ? (N > 1 ? N : 1) : (int)rsC;
        if (c_rows && (quick || (as_stored(M, K, rsA, csA, opA, lda) && as_stored(K, N, rsB, csB, opB, ldb))))
            return run(-1, opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, bias, act, 1, nullptr,
                       0, stream);
    }
    if (rsC == 1 && M > 1 && N > 1 && bias == nullptr) {
        // Column-major C: its transpose is row-major, C^T = B^T A^T (the same sums, so the
        // same results), with op(A) <- B^T and op(B) <- A^T.
        int opA, opB, lda, ldb;
        if (csC <= 0x7fffffffLL && as_stored(N, K, csB, rsB, opA, lda) && as_stored(K, M, csA, rsA, opB, ldb))
            return run(-1, opA, opB, N, M, K, alpha, B, lda, 0, A, ldb, 0, beta, C, (int)csC, 0, nullptr, act, 1,
                       nullptr, 0, stream);
    }
    sgemm_impl::StridedArgs p;
    p.M = M; p.N = N; p.K = K;
    p.alpha = alpha; p.beta = beta;
    p.A = A; p.B = B; p.C = C;
    p.bias = bias; p.act = act; p.fringe = 0;
    p.lda = rsA; p.ldb = rsB; p.ldc = rsC;
    p.strideA = p.strideB = p.strideC = 0;
    p.incA = csA; p.incB = csB; p.incC = csC;
    hipError_t e;
    if (K == 0 || alpha == 0.0f) {
        const int gx = cdiv64(N, 256) < 64 ? (int)cdiv64(N, 256) : 64;
        const int gy = M < 1024 ? M : 1024;
        hipLaunchKernelGGL(sgemm_impl::sgemm_scale, dim3(gx, gy, 1), dim3(256, 1), 0, stream, p);
        e = hipGetLastError();
    } else {
        if (cdiv64(M, 64) * cdiv64(N, 64) * 512ull > 0xFFFFFFFFull)
            return SGEMM_ERROR_TOO_LARGE;
        e = launch_strided(p, stream);
    }
    return e == hipSuccess ? 0 : (int)e;
}

static_assert(SGEMM_NOALLOC_SCRATCH_BYTES == kSkCounterBytes + 2ull * 256 * 128 * 128 * sizeof(float),
              "scratch holds the counters and two 128 x 128 partial tiles per compute unit");

__global__ void __launch_bounds__(256) zero_words(unsigned *p, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        p[i] = 0u;
}

// Device address of this device's copy of `scratch`. Host code must never pass the array's
// name to a kernel (on the host it is a stand-in, not a device address); the address comes
// from hipGetSymbolAddress, once per device with that device current. The first call on a
// device also queues a kernel on `stream` that zeroes the tile counters, ahead of any
// kernel that reads them (every stream-K call leaves them at zero again). Returns 0 or a
// positive hipError_t.
int scratch_for_current_device(void **out, hipStream_t stream)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mtx;
    static void *addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev < 0 || dev >= kMaxDevices)
        return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mtx);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
        hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, static_cast<unsigned *>(p),
                           (int)(kSkCounterBytes / sizeof(unsigned)));
        e = hipGetLastError();
        if (e != hipSuccess)
            return (int)e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return 0;
}

// The batched entry points with operand forms. Arguments keep the positions of
// sgemm_strided_batched_general up to strideC (16); `batch_pos` is where batch sits in the
// caller's signature (17 without bias and act, 19 with them).
int batched(int batch_pos, int config, int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
            long long strideA, const float *B, int ldb, long long strideB, float beta, float *C, int ldc,
            long long strideC, const float *bias, int act, int batch, void *stream)
{
    if (config < -1 || config >= kNumConfigs)
        return SGEMM_ERROR_BAD_CONFIG;
    const Arg bad = check_args(opA, opB, M, N, K, alpha, A, lda, B, ldb, C, ldc, act);
    if (bad != ARG_OK)
        return -kPosBatchedOp[bad];
    if (const int pos = check_batch(M, N, ldc, strideA, strideB, strideC, batch, 9, 12, 16, batch_pos))
        return -pos;
    if (M == 0 || N == 0 || batch == 0)
        return SGEMM_SUCCESS;
    if (config >= 0 && kConfigs[config].kind == KIND_SK)
        return SGEMM_ERROR_WORKSPACE;
    return run(config, opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, bias,
               act, batch, nullptr, 0, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb, float beta,
          float *C, int ldc, void *stream)
{
    return general(kPosPlain, -1, SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nullptr,
                   SGEMM_ACT_NONE, stream);
}

int sgemm_ex(int config, int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream)
{
    return general(kPosPlain, config, SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   nullptr, SGEMM_ACT_NONE, stream);
}

int sgemm_op(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
             int ldb, float beta, float *C, int ldc, void *stream)
{
    return general(kPosOp, -1, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, SGEMM_ACT_NONE,
                   stream);
}

int sgemm_bias_act(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                   int ldb, float beta, float *C, int ldc, const float *bias, int act, void *stream)
{
    return general(kPosFused, -1, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream);
}

int sgemm_general(int config, int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                  const float *B, int ldb, float beta, float *C, int ldc, const float *bias, int act,
                  void *stream)
{
    return general(kPosFused, config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream);
}

int sgemm_strided_batched(int M, int N, int K, float alpha, const float *A, int lda, long long strideA,
                          const float *B, int ldb, long long strideB, float beta, float *C, int ldc,
                          long long strideC, int batch, void *stream)
{
    const Arg bad = check_args(SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, B, ldb, C, ldc, SGEMM_ACT_NONE);
    if (bad != ARG_OK)
        return -kPosBatched[bad];
    if (const int pos = check_batch(M, N, ldc, strideA, strideB, strideC, batch, 7, 10, 14, 15))
        return -pos;
    if (M == 0 || N == 0 || batch == 0)
        return SGEMM_SUCCESS;
    return run(-1, SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
               strideC, nullptr, SGEMM_ACT_NONE, batch, nullptr, 0, static_cast<hipStream_t>(stream));
}

int sgemm_strided_batched_general(int config, int opA, int opB, int M, int N, int K, float alpha, const float *A,
                                  int lda, long long strideA, const float *B, int ldb, long long strideB,
                                  float beta, float *C, int ldc, long long strideC, const float *bias, int act,
                                  int batch, void *stream)
{
    return batched(19, config, opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                   bias, act, batch, stream);
}

int sgemm_strided_batched_op(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                             long long strideA, const float *B, int ldb, long long strideB, float beta, float *C,
                             int ldc, long long strideC, int batch, void *stream)
{
    return batched(17, -1, opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                   nullptr, SGEMM_ACT_NONE, batch, stream);
}

int sgemm_general_ws(int config, int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                     const float *B, int ldb, float beta, float *C, int ldc, const float *bias, int act,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (workspace == nullptr ? workspace_bytes != 0 : (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
        return -16;
    return general(kPosFused, config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream,
                   workspace, workspace_bytes);
}

int sgemm_strided(int M, int N, int K, float alpha, const float *A, long long rsA, long long csA, const float *B,
                  long long rsB, long long csB, float beta, float *C, long long rsC, long long csC,
                  const float *bias, int act, void *stream)
{
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    if (reads_ab && A == nullptr) return -5;
    if (rsA < 0) return -6;
    if (csA < 0) return -7;
    if (reads_ab && B == nullptr) return -8;
    if (rsB < 0) return -9;
    if (csB < 0) return -10;
    if (M > 0 && N > 0 && C == nullptr) return -12;
    if (rsC < 0) return -13;
    if (csC < 0) return -14;
    // Distinct entries of the M x N window at distinct addresses: one stride walks a row
    // (or column) without reaching the next one. An empty window has no constraint.
    if (M > 1 && N > 1) {
        const bool rows = csC >= 1 && rsC >= (long long)(N - 1) * csC + 1;
        const bool cols = rsC >= 1 && csC >= (long long)(M - 1) * rsC + 1;
        if (!rows && !cols) return -13;
    } else if (M > 1 && N == 1 && rsC < 1) {
        return -13;
    } else if (N > 1 && M == 1 && csC < 1) {
        return -14;
    }
    if (act != SGEMM_ACT_NONE && act != SGEMM_ACT_GELU_TANH) return -16;
    // Every element offset (i*rs + j*cs over the window) must fit the kernels' 64-bit
    // arithmetic with room to spare: at most 2^60 floats for each operand.
    auto extent_ok = [](int rows, int cols, long long rs, long long cs) {
        const unsigned __int128 e = (unsigned __int128)(rows > 0 ? rows - 1 : 0) * (unsigned long long)rs +
                                    (unsigned __int128)(cols > 0 ? cols - 1 : 0) * (unsigned long long)cs;
        return e < ((unsigned __int128)1 << 60);
    };
    if (reads_ab && !extent_ok(M, K, rsA, csA)) return -6;
    if (reads_ab && !extent_ok(K, N, rsB, csB)) return -9;
    if (M > 0 && N > 0 && !extent_ok(M, N, rsC, csC)) return -13;
    return strided(M, N, K, alpha, A, rsA, csA, B, rsB, csB, beta, C, rsC, csC, bias, act,
                   static_cast<hipStream_t>(stream));
}

int sgemm_general_noalloc(int config, int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                          const float *B, int ldb, float beta, float *C, int ldc, const float *bias, int act,
                          void *stream)
{
    if (config < -1 || config >= kNumConfigs)
        return SGEMM_ERROR_BAD_CONFIG;
    const Arg bad = check_args(opA, opB, M, N, K, alpha, A, lda, B, ldb, C, ldc, act);
    if (bad != ARG_OK)
        return -kPosFused[bad];
    if (M == 0 || N == 0)
        return SGEMM_SUCCESS;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (const int e = scratch_for_current_device(&ws, s))
        return e;
    // A forced stream-K configuration whose workspace exceeds the array returns
    // SGEMM_ERROR_WORKSPACE from run(); the automatic choice only considers those that fit.
    return run(config, opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, bias, act, 1, ws,
               SGEMM_NOALLOC_SCRATCH_BYTES, s);
}

size_t sgemm_workspace_size(int config)
{
    const int cus = device_cus();
    if (cus <= 0)
        return 0;
    size_t most = 0;
    for (int i = 0; i < kNumConfigs; ++i) {
        if (kConfigs[i].kind != KIND_SK || (config >= 0 && i != config))
            continue;
        const size_t b = sk_workspace_bytes(kConfigs[i], cus);
        most = b > most ? b : most;
    }
    return most;
}

int sgemm_select_config_ws(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                           const float *C, int ldc, size_t workspace_bytes)
{
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.0f)
        return -1;
    return choose(M, N, K, vector_ok(SGEMM_OP_N, SGEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc), workspace_bytes,
                  workspace_bytes > 0 ? device_cus() : 0);
}

int sgemm_select_config_general(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                                long long strideA, const float *B, int ldb, long long strideB, const float *C,
                                int ldc, long long strideC, int batch, size_t workspace_bytes)
{
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.0f || batch <= 0)
        return -1;
    const bool vec = vector_ok(opA != 0, opB != 0, M, N, K, A, lda, B, ldb, C, ldc) &&
                     (batch == 1 || (strideA % 4 == 0 && strideB % 4 == 0 && strideC % 4 == 0));
    return choose(M, N, K, vec, batch == 1 ? workspace_bytes : 0,
                  batch == 1 && workspace_bytes > 0 ? device_cus() : 0, batch);
}

int sgemm_config_count(void) { return kNumConfigs; }

const char *sgemm_config_name(int config)
{
    return (config >= 0 && config < kNumConfigs) ? kConfigs[config].name : nullptr;
}

const char *sgemm_config_describe(int config)
{
    // One line per configuration, written once (thread-safe static initialisation).
    struct Lines {
        char text[kNumConfigs][320];
        Lines()
        {
            static const char *const kinds[] = {"tile16", "mfma", "streamk", "valu"};
            for (int i = 0; i < kNumConfigs; ++i) {
                const Config &c = kConfigs[i];
                const bool mfma = c.kind == KIND_MFMA || c.kind == KIND_SK;
                const char *loader = c.kind == KIND_TILE16 ? "staged-elementwise"
                                     : c.kind == KIND_VALU ? "staged-k-major"
                                     : c.dma               ? "direct-16B"
                                                           : "staged-16B";
                const char *unaligned = !mfma                             ? loader
                                        : c.unaligned_dma                   ? "direct-16B-unaligned"
                                        : c.kind == KIND_SK                 ? "data-parallel-staged-4B"
                                                                            : "staged-4B";
                snprintf(text[i], sizeof(text[i]),
                         "name=%s kind=%s tile=%dx%dx%d waves=%dx%d kgroups=%d threads=%d ahead=%d loader=%s "
                         "lds_bytes=%d band=%d unaligned=%s unaligned_bk=%d compute=%s",
                         c.name, kinds[c.kind], c.bm, c.bn, c.bk, c.wgm, c.wgn, c.wgk, c.threads, c.pf, loader,
                         c.lds_bytes, c.group_m, unaligned, c.unaligned_bk,
                         !mfma ? "v_fma_f32" : c.mb == 16 ? "v_mfma_f32_16x16x4_f32" : "v_mfma_f32_32x32x2_f32");
            }
        }
    };
    static const Lines lines;
    return (config >= 0 && config < kNumConfigs) ? lines.text[config] : nullptr;
}

int sgemm_select_config(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                        const float *C, int ldc)
{
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.0f)
        return -1;
    return choose(M, N, K, vector_ok(SGEMM_OP_N, SGEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc));
}

int sgemm_launch_shape(int config, int M, int N, int K, int grid[3], int block[3])
{
    if (config < 0 || config >= kNumConfigs) return SGEMM_ERROR_BAD_CONFIG;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const Config &c = kConfigs[config];
    if (c.kind == KIND_TILE16) {
        grid[0] = (int)cdiv64(N, 16); grid[1] = (int)cdiv64(M, 16); grid[2] = 1;
        block[0] = 16; block[1] = 16; block[2] = 1;
        return 0;
    }
    const uint64_t tiles = tile_count(c, M, N);
    if (c.kind == KIND_SK) {
        // The split of a 256-CU device (MI355X): whole-tile rounds (direct-copy
        // configurations), then one workgroup per CU (at most one per K-tile step) for the
        // shared tiles.
        if (!sk_work_fits(c, M, N, K, 256)) return SGEMM_ERROR_TOO_LARGE;
        int dp = 0;
        grid[0] = sk_split((int)tiles, (int)cdiv64(K, c.bk), 256, c.dma, dp); grid[1] = 1; grid[2] = 1;
        block[0] = c.threads; block[1] = 1; block[2] = 1;
        return 0;
    }
    const uint64_t wgs = grid_count(c, M, N, fringe_cols(c, M, N, K, 1));
    if (wgs * (uint64_t)c.threads > 0xFFFFFFFFull) return SGEMM_ERROR_TOO_LARGE;
    grid[0] = (int)wgs; grid[1] = 1; grid[2] = 1;
    block[0] = c.threads; block[1] = 1; block[2] = 1;
    return 0;
}

const char *sgemm_status_string(int status)
{
    switch (status) {
    case 0: return "success";
    case SGEMM_ERROR_TOO_LARGE: return "problem too large: the tile grid exceeds one launch";
    case SGEMM_ERROR_BAD_CONFIG: return "configuration id out of range";
    case SGEMM_ERROR_WORKSPACE: return "stream-K configuration without a large enough workspace";
    default: break;
    }
    if (status < 0 && status >= -20) {
        static const char *const msgs[21] = {
            "", "invalid argument 1", "invalid argument 2", "invalid argument 3", "invalid argument 4",
            "invalid argument 5", "invalid argument 6", "invalid argument 7", "invalid argument 8",
            "invalid argument 9", "invalid argument 10", "invalid argument 11", "invalid argument 12",
            "invalid argument 13", "invalid argument 14", "invalid argument 15", "invalid argument 16",
            "invalid argument 17", "invalid argument 18", "invalid argument 19", "invalid argument 20"};
        return msgs[-status];
    }
    if (status > 0)
        return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}

const char *sgemm_version(void) { return "tiled_fp32_gemm_02_amd 0.2 (gfx950)"; }

}  // extern "C"
