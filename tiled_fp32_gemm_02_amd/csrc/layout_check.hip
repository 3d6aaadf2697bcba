// Host-side check of the direct-copy LDS layouts (TileDMA) of every direct-copy
// configuration, in every operand form and copy width, run without a GPU.
//
// For each tile it checks, with the same index functions the kernels use:
//  - every copy instruction of every wave lands a whole chunk (or float) of the tile at
//    the LDS position the layout gives that chunk;
//  - the copies together cover every element of the tile exactly once;
//  - the layout maps the tile one-to-one onto its SIZE floats of LDS;
//  - the fragment reads of the matrix-core loop (16-byte reads of k-contiguous rows,
//    1-, 2- or 4-float reads of m- or n-contiguous rows, one float per block where plain
//    B's blocks sit side by side) meet no LDS bank conflict in a
//    model of the 64-bank LDS that serves 64 dwords per pass (64 lanes of a 4-byte read,
//    32 of an 8-byte one, 16 of a 16-byte one). The hardware counters are the final
//    word on conflicts; this catches a layout that cannot be conflict-free;
//  - on rows only 4-byte aligned (TileDMA's U form), with the kernels' own copy plans
//    over every tile and K-tile of a set of odd-sized operands: each 16-byte copy of a
//    K-tile that does not hold the end of K reads inside the operand, and the 4-byte
//    copies of the K-tile that does read only elements of the matrix.
// Prints one line per failure and exits non-zero if any check fails.
#include <cstdio>
#include <cstring>
#include <type_traits>
#include <vector>

#include "sgemm_configs.inc"
#include "sgemm_kernels.hpp"

using namespace sgemm_impl;

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            if (failures < 50) {                          \
                std::printf(__VA_ARGS__);                 \
                std::printf("\n");                        \
            }                                             \
            ++failures;                                   \
        }                                                 \
    } while (0)

template <class T, int TR, int TC, int NT, bool KC, int VW>
static void check_copies(const char *what)
{
    std::vector<int> hits(TR * TC, 0);
    for (int w = 0; w < NT / 64; ++w)
        for (int c = 0; c < T::CH; ++c) {
            const int first = w * 64 + c * NT;
            for (int l = 0; l < 64; ++l) {
                int r, col;
                T::where(c, w * 64 + l, r, col);
                const int slot = first + l;
                CHECK(r >= 0 && r < TR && col >= 0 && col + VW <= TC && col % VW == 0,
                      "%s: slot %d -> (%d, %d) outside the tile", what, slot, r, col);
                if (!(r >= 0 && r < TR && col >= 0 && col + VW <= TC))
                    continue;
                for (int v = 0; v < VW; ++v) {
                    CHECK(T::elem(r, col + v) == slot * VW + v, "%s: slot %d element (%d, %d) at %d, copy writes %d",
                          what, slot, r, col + v, T::elem(r, col + v), slot * VW + v);
                    ++hits[r * TC + col + v];
                }
            }
        }
    for (int i = 0; i < TR * TC; ++i)
        CHECK(hits[i] == 1, "%s: element (%d, %d) copied %d times", what, i / TC, i % TC, hits[i]);
    std::vector<int> seen(TR * TC, 0);
    for (int r = 0; r < TR; ++r)
        for (int col = 0; col < TC; ++col) {
            const int e = T::elem(r, col);
            CHECK(e >= 0 && e < TR * TC, "%s: (%d, %d) at %d, outside %d floats", what, r, col, e, TR * TC);
            if (e >= 0 && e < TR * TC)
                ++seen[e];
        }
    for (int i = 0; i < TR * TC; ++i)
        CHECK(seen[i] == 1, "%s: LDS float %d holds %d elements", what, i, seen[i]);
}

// One LDS read instruction of a wave: lane l reads `width` floats starting at addr[l].
// Lanes are served in passes of 64 / width; within a pass no two lanes may touch the
// same bank at different addresses.
static void check_read(const char *what, const int *addr, int width)
{
    const int per_pass = 64 / width;
    for (int p0 = 0; p0 < 64; p0 += per_pass) {
        int owner[64];
        for (int b = 0; b < 64; ++b)
            owner[b] = -1;
        for (int l = p0; l < p0 + per_pass; ++l)
            for (int v = 0; v < width; ++v) {
                const int a = addr[l] + v, bank = a & 63;
                CHECK(owner[bank] < 0 || owner[bank] == a, "%s: lanes of one pass meet at bank %d (floats %d, %d)",
                      what, bank, owner[bank], a);
                owner[bank] = a;
            }
    }
}

// The U form's reads for one operand stored as `rows` x `cols` floats with row stride ld,
// cut into tiles of TR x TC as the kernels cut it (KC: rows run along m or n and columns
// along k, else rows along k). Every tile and K-tile is walked with the kernel's own copy
// plan (T::plan, and the 4-byte layout T::Words in the K-tile holding the end of K).
template <class T, int TR, int TC, int NT, bool KC>
static void check_u_reads(const char *what, int rows, int cols, int64_t ld)
{
    const int mdim = KC ? rows : cols, K = KC ? cols : rows;
    const int tmn = KC ? TR : TC, kext = KC ? TC : TR;
    const int64_t extent = (int64_t)(rows - 1) * ld + cols;     // floats of the operand
    for (int t = 0; t * tmn < mdim; ++t)
        for (int kt = 0; kt * kext < K; ++kt) {
            const int mn = mdim - t * tmn, k = K - kt * kext;
            const int64_t origin = KC ? (int64_t)t * TR * ld + (int64_t)kt * TC : (int64_t)kt * TR * ld + (int64_t)t * TC;
            for (int tid = 0; tid < NT; ++tid) {
                if (k > kext) {
                    const typename T::Lane L = T::template plan<true>(ld, mn, tid);
                    for (int c = 0; c < T::CH; ++c) {
                        if (L.off[c] == 0x80000000u)
                            continue;
                        const int64_t f = origin + L.off[c] / 4;
                        CHECK(f >= 0 && f + 4 <= extent, "%s: %dx%d ld %lld tile %d K-tile %d thread %d copy %d reads "
                              "floats %lld..%lld of %lld", what, rows, cols, (long long)ld, t, kt, tid, c,
                              (long long)f, (long long)f + 3, (long long)extent);
                    }
                } else {
                    using W = typename T::Words;
                    for (int c = 0; c < W::CH; ++c) {
                        int r, col;
                        W::where(c, tid, r, col);
                        if (!((KC ? r : col) < mn && (KC ? col : r) < k))
                            continue;               // not copied: reads as zero
                        const int64_t sr = (KC ? (int64_t)t * TR : (int64_t)kt * TR) + r;
                        const int64_t sc = (KC ? (int64_t)kt * TC : (int64_t)t * TC) + col;
                        CHECK(sr < rows && sc < cols, "%s: %dx%d ld %lld tile %d last K-tile thread %d word %d reads "
                              "(%lld, %lld)", what, rows, cols, (long long)ld, t, tid, c, (long long)sr, (long long)sc);
                    }
                }
            }
        }
}

// Odd-sized operands for check_u_reads: extents around one and two tiles along each
// dimension, packed and padded row strides, and the shortest strides the host allows.
template <class T, int TR, int TC, int NT, bool KC>
static void check_u_operand(const char *what)
{
    const int dims[][2] = {{2 * TR + 3, 2 * TC + 1}, {TR - 1, TC + 5}, {1, 4 * TC + 3}, {3, 5}, {TR + 1, 1}};
    for (const auto &d : dims)
        for (int pad : {0, 3}) {
            const int64_t ld = d[1] + pad < 4 ? 4 : d[1] + pad;
            check_u_reads<T, TR, TC, NT, KC>(what, d[0], d[1], ld);
        }
}

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int MB, bool TA, bool TB, int VW>
static void check_config(const char *name)
{
    using T = MfmaTile<BM, BN, BK, WGM, WGN, WGK, 1, true, TA, TB, true, false, MB>;
    using TU = MfmaTile<BM, BN, BK, WGM, WGN, WGK, 1, true, TA, TB, false, true, MB>;
    // VW = 4: the 16-byte copies; VW = 1: the 4-byte layout of the same tiles
    using A = typename std::conditional<VW == 4, typename T::AIO, typename T::AIO::Words>::type;
    using B = typename std::conditional<VW == 4, typename T::BIO, typename T::BIO::Words>::type;
    static_assert(std::is_same<typename TU::AIO::Words, typename T::AIO::Words>::value &&
                  std::is_same<typename TU::BIO::Words, typename T::BIO::Words>::value, "one 4-byte layout");
    char what[160];
    std::snprintf(what, sizeof what, "%s %s%s VW=%d A", name, TA ? "t" : "n", TB ? "t" : "n", VW);
    check_copies<A, TA ? BK : BM, TA ? BM : BK, T::NT, !TA, VW>(what);
    std::snprintf(what, sizeof what, "%s %s%s VW=%d B", name, TA ? "t" : "n", TB ? "t" : "n", VW);
    check_copies<B, TB ? BN : BK, TB ? BK : BN, T::NT, TB, VW>(what);
    if constexpr (VW == 4) {
        std::snprintf(what, sizeof what, "%s %s%s unaligned A", name, TA ? "t" : "n", TB ? "t" : "n");
        check_u_operand<typename TU::AIO, TA ? BK : BM, TA ? BM : BK, T::NT, !TA>(what);
        std::snprintf(what, sizeof what, "%s %s%s unaligned B", name, TA ? "t" : "n", TB ? "t" : "n");
        check_u_operand<typename TU::BIO, TB ? BN : BK, TB ? BK : BN, T::NT, TB>(what);
    }

    // The loop's fragment reads, per wave and group of KGRP k (as in MfmaTile::read_frag):
    // lane l is row/column l % MB of its block and supplies k = 4 * (l / MB) + step.
    constexpr int TM = T::TM, TN = T::TN, KS = T::KSLICE, KG = T::KGRP;
    for (int wave = 0; wave < T::NT / 64; ++wave) {
        const int wk = wave / (WGM * WGN), wm = (wave % (WGM * WGN)) / WGN, wn = wave % WGN;
        for (int g = 0; g < KS / KG; ++g) {
            int addr[64];
            if (!TA) {
                for (int a = 0; a < TM; ++a) {
                    for (int l = 0; l < 64; ++l)
                        addr[l] = A::elem(wm * T::WTM + (l % MB) + a * MB, wk * KS + KG * g + 4 * (l / MB));
                    std::snprintf(what, sizeof what, "%s %s%s VW=%d A read (wave %d, group %d, block %d)", name,
                                  TA ? "t" : "n", TB ? "t" : "n", VW, wave, g, a);
                    check_read(what, addr, 4);
                }
            } else {
                for (int s = 0; s < 4; ++s) {
                    for (int l = 0; l < 64; ++l)
                        addr[l] = A::elem(wk * KS + KG * g + 4 * (l / MB) + s, wm * T::WTM + (l % MB) * TM);
                    std::snprintf(what, sizeof what, "%s %s%s VW=%d A read (wave %d, group %d, k %d)", name,
                                  TA ? "t" : "n", TB ? "t" : "n", VW, wave, g, s);
                    check_read(what, addr, TM);
                }
            }
            if (TB) {
                for (int b = 0; b < TN; ++b) {
                    for (int l = 0; l < 64; ++l)
                        addr[l] = B::elem(wn * T::WTN + (l % MB) + b * MB, wk * KS + KG * g + 4 * (l / MB));
                    std::snprintf(what, sizeof what, "%s %s%s VW=%d B read (wave %d, group %d, block %d)", name,
                                  TA ? "t" : "n", TB ? "t" : "n", VW, wave, g, b);
                    check_read(what, addr, 4);
                }
            } else if (T::BSIDE) {
                for (int s = 0; s < 4; ++s)
                    for (int b = 0; b < TN; ++b) {
                        for (int l = 0; l < 64; ++l)
                            addr[l] = B::elem(wk * KS + KG * g + 4 * (l / MB) + s, wn * T::WTN + (l % MB) + b * MB);
                        std::snprintf(what, sizeof what, "%s %s%s VW=%d B read (wave %d, group %d, k %d, block %d)",
                                      name, TA ? "t" : "n", TB ? "t" : "n", VW, wave, g, s, b);
                        check_read(what, addr, 1);
                    }
            } else {
                for (int s = 0; s < 4; ++s) {
                    for (int l = 0; l < 64; ++l)
                        addr[l] = B::elem(wk * KS + KG * g + 4 * (l / MB) + s, wn * T::WTN + (l % MB) * TN);
                    std::snprintf(what, sizeof what, "%s %s%s VW=%d B read (wave %d, group %d, k %d)", name,
                                  TA ? "t" : "n", TB ? "t" : "n", VW, wave, g, s);
                    check_read(what, addr, TN);
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int MB>
static int check_all_forms(const char *name)
{
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, false, false, 4>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, false, true, 4>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, true, false, 4>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, true, true, 4>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, false, false, 1>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, false, true, 1>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, true, false, 1>(name);
    check_config<BM, BN, BK, WGM, WGN, WGK, MB, true, true, 1>(name);
    return 1;
}

template <bool DMA, int BM, int BN, int BK, int WGM, int WGN, int WGK, int MB>
static int check_if_direct(const char *name)
{
    if constexpr (DMA)
        return check_all_forms<BM, BN, BK, WGM, WGN, WGK, MB>(name);
    else
        return 0;
}

int main()
{
    int configs = 0;
#define SGEMM_CHECK(name, BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB) \
    configs += check_if_direct<(DMA != 0), BM, BN, BK, WGM, WGN, WGK, MB>(name);
    SGEMM_MFMA_CONFIGS(SGEMM_CHECK)
    SGEMM_SK_CONFIGS(SGEMM_CHECK)
#undef SGEMM_CHECK
    std::printf("layout_check: %d direct-copy configurations x 8 forms, %d failures\n", configs, failures);
    return failures == 0 ? 0 : 1;
}
