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
//    word on conflicts; this catches a layout that cannot be conflict-free.
// Prints one line per failure and exits non-zero if any check fails.
#include <cstdio>
#include <cstring>
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

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int MB, bool TA, bool TB, int VW>
static void check_config(const char *name)
{
    using T = MfmaTile<BM, BN, BK, WGM, WGN, WGK, 1, true, TA, TB, VW == 4, false, MB>;
    using A = typename T::AIO;
    using B = typename T::BIO;
    char what[160];
    std::snprintf(what, sizeof what, "%s %s%s VW=%d A", name, TA ? "t" : "n", TB ? "t" : "n", VW);
    check_copies<A, TA ? BK : BM, TA ? BM : BK, T::NT, !TA, VW>(what);
    std::snprintf(what, sizeof what, "%s %s%s VW=%d B", name, TA ? "t" : "n", TB ? "t" : "n", VW);
    check_copies<B, TB ? BN : BK, TB ? BK : BN, T::NT, TB, VW>(what);

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
