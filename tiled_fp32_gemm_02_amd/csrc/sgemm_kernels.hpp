// Device kernels for row-major fp32 C = act(alpha*op(A)*op(B) + beta*C + bias) on
// gfx950 (MI355X). op is the identity or a transpose; bias (per column) and act (none
// or tanh-form GELU) are optional and off for the plain product.
//
// This header holds the matrix-core kernels, sgemm_mfma (one workgroup per output tile)
// and sgemm_mfma_sk (stream-K: equal shares of the tiles x K-tiles work per compute
// unit), and the helpers shared with the kernels in sgemm_aux_kernels.hpp (16x16
// baseline, vector-ALU micro-tile, quick-return scaling).
// sgemm_mfma is the hot path. A workgroup owns a BM x BN tile of C; each wave owns
//    a (BM/WGM) x (BN/WGN) sub-tile made of 32x32 blocks computed with the CDNA fp32
//    matrix instruction (32x32 outputs, 2 k-steps per issue), or of 16x16 blocks (4
//    k-steps per issue) for small, skinny and ragged products. A and B tiles reach a
//    ring of LDS stages with one barrier per K-tile: copied from HBM straight into LDS
//    (TileDMA; 16-byte copies, with 4-byte ones in the K-tile holding the end of K
//    when rows are only 4-byte aligned), or
//    staged through registers (TileIO). The next K-tile's loads (two with register
//    staging and PF = 2) are in flight while the current one is multiplied.
//
// Techniques from the pages and where they come from:
//  - Tiling through local memory so each global element is fetched once per
//    workgroup instead of once per thread (AutoMine++ #4, "Current algorithm";
//    GPT-2 post, "Tiled matrix multiplication").
//  - Thread coarsening with an outer-product update of a register tile
//    (AutoMine++ #4, "Use registers" and "Matrix product by outer products"); here
//    the register tile is the matrix-core accumulator and the outer products of
//    2-deep k slices are what each matrix instruction adds.
//  - Rectangular tiles and wide chunk loads, with a flat thread-to-chunk map in
//    which surplus threads idle (AutoMine++ #7, "Rectangular tiling" and "Fine
//    tuning"); double buffering with register staging and one barrier per step
//    (AutoMine++ #7, "Rectangular tiling"; Micro_gemm_4x4, "Pipeline (double
//    buffering)").
//  - Zero-filled out-of-range loads, a ceil-divided grid and predicated stores
//    (Micro_gemm_4x4, "A/B tile load" and "Final C write"; GPT-2 post, "Tiled matrix
//    multiplication").
//  - alpha/beta epilogue that skips reading C when beta is zero (Micro_gemm_4x4,
//    "Final C write (alpha, beta)").
//  - Transposed operands read in place, as the GPT-2 post's kernel takes transposed
//    views ("Tiled matrix multiplication"); bias and GELU applied to the product as in
//    its linear layers ("The whole model as one kernel", "From loops to kernels").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sgemm_impl {

typedef float floatx16 __attribute__((ext_vector_type(16)));
// Four floats at an address that is only 4-byte aligned (same registers as floatx4).
typedef float floatx4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

enum Act { ACT_NONE = 0, ACT_GELU_TANH = 1 };

struct GemmArgs {
    int M, N, K;
    float alpha, beta;
    const float *A;             // op(A) is M x K: A[i*lda + k], or A[k*lda + i] when transposed
    const float *B;             // op(B) is K x N: B[k*ldb + j], or B[j*ldb + k] when transposed
    float *C;
    const float *bias;          // N entries (one per column) or null
    int act;                    // Act
    int fringe;                 // last columns of C left to the fringe workgroups (see sgemm_mfma)
    int64_t lda, ldb, ldc;
    int64_t strideA, strideB, strideC;  // per blockIdx.z (batched form); 0 otherwise
};

// Arguments of the general-stride kernels (and of the C-scaling kernel, which serves both
// forms): the column strides as well (A(i,k) = A[i*lda + k*incA], B(k,j) = B[k*ldb + j*incB],
// C(i,j) = C[i*ldc + j*incC]). The tile kernels keep the smaller GemmArgs.
struct StridedArgs : GemmArgs {
    int64_t incA, incB, incC;
};

// ceil(a / b) for a >= 0, b >= 1, in unsigned arithmetic so that a near 2^31 does not overflow.
__device__ __forceinline__ int ceil_div(int a, int b) { return (int)(((unsigned)a + (unsigned)b - 1u) / (unsigned)b); }

// tanh-form GELU in fp32: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
__device__ __forceinline__ float gelu_tanh(float x)
{
    const float c = 0.7978845608028654f;    // sqrt(2/pi)
    return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

// The epilogue value of one entry: act(alpha*acc + beta*c + bias_j); c is read only
// when beta != 0.
__device__ __forceinline__ float finish(float acc, float alpha, float beta, const float *cptr,
                                        const float *bias, int j, int act)
{
    float out = alpha * acc;
    if (beta != 0.f)
        out += beta * *cptr;
    if (bias)
        out += bias[j];
    if (act == ACT_GELU_TANH)
        out = gelu_tanh(out);
    return out;
}

// The same value with C's entry already loaded (c, used only when beta != 0) and the
// bias entry bj (used only when has_bias), in the same order of operations.
__device__ __forceinline__ float finish_value(float acc, float alpha, float beta, float c, bool has_bias,
                                              float bj, int act)
{
    float out = alpha * acc;
    if (beta != 0.f)
        out += beta * c;
    if (has_bias)
        out += bj;
    if (act == ACT_GELU_TANH)
        out = gelu_tanh(out);
    return out;
}

// Map the linear workgroup id to a (tile_m, tile_n) pair.
//
// Workgroups are handed to the 8 XCDs in round-robin order of their id, and each
// XCD has its own L2. The first step renumbers ids so that each XCD receives one
// contiguous range of the logical order. The second walks that order in groups of
// `group_m` tile rows, column by column, so workgroups that run together share A
// row panels and B column panels in L2.
// Workgroup id -> position in a launch order where each of the 8 XCDs (which take ids
// round-robin) receives one contiguous range.
__device__ __forceinline__ int xcd_contiguous(int wg, int total)
{
    constexpr int XCDS = 8;
    const int per = total / XCDS, rem = total % XCDS;
    const int xcd = wg % XCDS, slot = wg / XCDS;
    return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Position in the launch order -> (tile_m, tile_n), walking bands of `group_m` tile rows
// column by column.
__device__ __forceinline__ void band_coords(int logical, int tiles_m, int tiles_n, int group_m, int &tm, int &tn)
{
    const int band = group_m * tiles_n;
    const int first_m = (logical / band) * group_m;
    const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in_band = logical % band;
    tm = first_m + in_band % rows;
    tn = in_band / rows;
}

__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn)
{
    band_coords(xcd_contiguous(wg, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
}

// One operand tile as it sits in memory: TR rows of TC contiguous floats (row stride
// ld), copied HBM -> registers -> LDS in 4-float chunks. Thread t takes chunks
// t, t + NT, ...; consecutive threads take consecutive chunks along a row, and when
// the tile has fewer chunks than threads the surplus threads idle. The LDS copy keeps
// the same layout, with 4 floats of padding after every G rows, G = 64 / TC for rows
// of 16 or 32 floats and G = 1 for longer rows. Then the G rows that one group of 16
// lanes stores with 128-bit writes fill the 64 LDS banks exactly once, and 16
// consecutive rows read at one column (a fragment read) start in 16 distinct 4-bank
// groups. (The bank-conflict counter confirms this on gfx950: a plain 4-float row
// padding leaves the stores of 16-float rows colliding two ways.)
template <int TR, int TC, int NT>
struct TileIO {
    static constexpr int CPR = TC / 4;
    static constexpr int CHUNKS = TR * TC / 4;
    static constexpr int CH = (CHUNKS + NT - 1) / NT;
    static constexpr bool IDLE = CHUNKS % NT != 0;
    static constexpr int G = TC >= 64 ? 1 : 64 / TC;       // rows per 4-float pad
    static constexpr int SIZE = TR * TC + (TR / G) * 4;
    static_assert(TC % 16 == 0, "rows are multiples of 16 floats");
    static_assert(TR % G == 0, "whole groups of rows");

    // Offset (floats) of row r, and of element (r, col), of the tile in LDS.
    __device__ __forceinline__ static int row(int r) { return r * TC + (r / G) * 4; }
    __device__ __forceinline__ static int elem(int r, int col) { return row(r) + col; }

    // src points at the tile origin; rows/cols are how many rows and columns from the
    // origin lie inside the matrix. VEC: 128-bit loads (row starts 16-byte aligned and
    // the column extent a multiple of 4, so a chunk is wholly in or out); otherwise every
    // float is checked. EDGE = false promises the whole tile is inside. STRIDED: the
    // columns lie `inc` floats apart (a general-stride operand), read float by float.
    template <bool VEC, bool EDGE, bool STRIDED = false>
    __device__ __forceinline__ static void load(floatx4 (&r)[CH], const float *__restrict__ src, int64_t ld,
                                                int rows, int cols, int tid, int64_t inc = 1)
    {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            if (IDLE && idx >= CHUNKS)
                break;
            const int rr = idx / CPR, cc = (idx % CPR) * 4;
            const float *p = src + (int64_t)rr * ld + (STRIDED ? (int64_t)cc * inc : (int64_t)cc);
            if constexpr (STRIDED) {
                const bool rok = rr < rows;
                r[c].x = (!EDGE || (rok && cc + 0 < cols)) ? p[0] : 0.f;
                r[c].y = (!EDGE || (rok && cc + 1 < cols)) ? p[inc] : 0.f;
                r[c].z = (!EDGE || (rok && cc + 2 < cols)) ? p[2 * inc] : 0.f;
                r[c].w = (!EDGE || (rok && cc + 3 < cols)) ? p[3 * inc] : 0.f;
            } else if (VEC) {
                if (!EDGE || (rr < rows && cc < cols))
                    r[c] = *reinterpret_cast<const floatx4 *>(p);
                else
                    r[c] = floatx4{0.f, 0.f, 0.f, 0.f};
            } else {
                // Rows only 4-byte aligned: a chunk wholly inside is still one 16-byte
                // load (global memory takes dword-aligned vector accesses); the chunk that
                // straddles the end of a row, or lies outside, is read float by float.
                const bool rok = rr < rows;
                if (!EDGE || (rok && cc + 3 < cols)) {
                    r[c] = *reinterpret_cast<const floatx4u *>(p);
                } else {
                    r[c].x = (rok && cc + 0 < cols) ? p[0] : 0.f;
                    r[c].y = (rok && cc + 1 < cols) ? p[1] : 0.f;
                    r[c].z = (rok && cc + 2 < cols) ? p[2] : 0.f;
                    r[c].w = (rok && cc + 3 < cols) ? p[3] : 0.f;
                }
            }
        }
    }

    struct Lane {};     // register staging keeps no per-lane copy plan
    template <bool EDGE>
    __device__ __forceinline__ static Lane plan(int64_t, int, int) { return Lane{}; }

    __device__ __forceinline__ static void store(const floatx4 (&r)[CH], float *lds, int tid)
    {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            if (IDLE && idx >= CHUNKS)
                break;
            *reinterpret_cast<floatx4 *>(&lds[row(idx / CPR) + (idx % CPR) * 4]) = r[c];
        }
    }
};

typedef __attribute__((address_space(3))) void lds_void;

// The same operand tile copied HBM -> LDS directly, with no staging registers, by
// buffer loads into LDS: one such instruction of one wave fills 64 consecutive LDS
// slots of VW floats, lane l the l-th (VW = 4: 16-byte copies, for rows that are
// 16-byte aligned; VW = 1: 4-byte copies, for rows that are only 4-byte aligned; both
// lane layouts were checked on the GPU with a probe). The tile is TR rows of TC floats
// with no padding, in 16-byte chunks; inside row r, chunk c sits in chunk slot
// c ^ swz(r). A lane fetches whichever global data belongs in its slot, so the copy
// stays contiguous while the reads stay free of bank conflicts on the 64-bank LDS:
//  - KCONTIG (rows run along k: plain A, transposed B): 16 consecutive rows read at one
//    chunk land in 16 distinct 4-bank groups;
//  - otherwise (rows run along m or n): consecutive lanes read consecutive chunks of one
//    row, and rows 4 apart (the two half-waves) use opposite halves of each 16-slot window.
//    A row of only 8 chunks (a 32-wide tile) fills half the banks, so there the rows
//    themselves are permuted instead: logical row r sits at row r ^ ((r >> 2) & 1), which
//    puts rows 4 apart in opposite halves of the banks.
// Data outside the matrix is fetched at an offset past the buffer's range, which the
// hardware answers with zeros, so partial tiles arrive zero-padded as in TileIO: per
// chunk for VW = 4 (the extents are then multiples of 4), per float for VW = 1.
// Needs row strides below 2^20 floats (every byte offset from the tile origin stays
// below 2^31 for TR <= 256).
//
// Q16 (only for m- or n-contiguous tiles): the tile is read by 16x16-block matrix code one
// float per lane, so four groups of 16 lanes read rows k, k+4, k+8 and k+12 at the same 16
// columns in one pass. Row r's chunks are then XORed with ((r >> 2) & 3) << 2, which puts
// those four rows' 16 columns in four distinct 16-bank groups. With 32-wide rows (row
// permutation, the two halves of the banks) the chunks are XORed with ((r >> 3) & 1) << 2
// instead: rows 4 apart alternate halves through the permutation, rows 8 apart alternate
// 16-column groups through the XOR, so the four rows again meet four distinct groups.
//
// Panels (PW < TC, m- or n-contiguous tiles only): rows of 3 * 2^j floats (48, 96) have no
// such swizzle, so the tile is kept as TC / PW panels of TR rows x PW columns, one after
// the other, each laid out as a TR x PW tile of its own. A read of 16 or 32 consecutive
// columns that stays inside one panel then meets the banks exactly as in a PW-wide tile.
//
// U (VW = 4, rows only 4-byte aligned): 16-byte copies from 4-byte aligned addresses
// (global memory takes dword-aligned vector accesses, as the register-staged loads also
// rely on). A chunk then always holds the 4 floats it names, but a chunk that crosses the
// end of a row brings floats of the next row along. That is harmless along m or n (they
// land in tile columns or rows past the matrix edge, whose outputs are never written),
// but not along k, and the last row's crossing chunk would read past the operand. So the
// K-tile that holds the end of K is copied in 4-byte words (the VW = 1 layout, `Words`)
// with every float checked, and every other K-tile ends at least one row before the
// operand's last row, whose row stride (at least 4 floats, checked by the host) keeps a
// crossing chunk inside the operand.
template <int TR, int TC, int NT, bool KCONTIG, int VW, bool Q16 = false, int PW = TC, bool U = false>
struct TileDMA {
    static constexpr int NP = TC / PW;                  // panels
    static constexpr int CPR = PW / 4;                  // chunks per row of a panel
    static constexpr int PSIZE = TR * PW;
    static constexpr int SLOTS = TR * TC / VW;
    static constexpr int CH = SLOTS / NT;               // copy instructions per thread
    static constexpr int SIZE = TR * TC;
    static_assert(VW == 4 || VW == 1, "16- or 4-byte copies");
    static_assert(!U || VW == 4, "16-byte copies on 4-byte aligned rows");
    static constexpr int KEXT = KCONTIG ? TC : TR;      // the tile's extent along k
    static_assert(NT % 64 == 0 && SLOTS % NT == 0, "whole copy instructions per wave");
    static_assert(TC % PW == 0 && (NP == 1 || !KCONTIG), "whole panels, along m or n only");
    static_assert(CPR == 4 || CPR == 8 || CPR % 16 == 0, "slot swizzle needs these row lengths");

    static constexpr bool ROWPERM = !KCONTIG && CPR == 8;
    // Rows of 16 floats (a 16-wide tile, read by 16x16-block code) fill a quarter of the
    // banks: rows are permuted within groups of four, logical row r at r ^ ((r >> 2) & 3),
    // so the four rows k, k+4, k+8, k+12 that one pass reads sit in four distinct quarters.
    static constexpr bool ROWPERM4 = !KCONTIG && CPR == 4;
    static_assert(!ROWPERM || TR % 2 == 0, "row pairs");
    static_assert(!ROWPERM4 || TR % 4 == 0, "row quads");
    __host__ __device__ __forceinline__ static int swz(int r)
    {
        if (KCONTIG)
            return CPR >= 16 ? (r & 15) : ((r / (16 / CPR)) & (CPR - 1));
        if (ROWPERM4)
            return 0;
        if (ROWPERM)
            return Q16 ? ((r >> 3) & 1) << 2 : 0;
        return Q16 ? ((r >> 2) & 3) << 2 : ((r >> 2) & 1) << 3;
    }
    // Physical row of logical row r (an involution: it also maps physical to logical).
    __host__ __device__ __forceinline__ static int prow(int r)
    {
        return ROWPERM ? (r ^ ((r >> 2) & 1)) : ROWPERM4 ? (r ^ ((r >> 2) & 3)) : r;
    }
    __host__ __device__ __forceinline__ static int elem(int r, int col)
    {
        if constexpr (NP == 1) {
            return 4 * (prow(r) * CPR + ((col >> 2) ^ swz(r))) + (col & 3);
        } else {
            const int p = col / PW, c = col % PW;
            return p * PSIZE + 4 * (prow(r) * CPR + ((c >> 2) ^ swz(r))) + (c & 3);
        }
    }

    // Row and column, inside the tile, of the first float that copy c brings to this lane.
    __host__ __device__ __forceinline__ static void where(int c, int tid, int &r, int &col)
    {
        const int f = ((tid >> 6) * 64 + c * NT + (tid & 63)) * VW;   // its LDS position
        const int p = NP == 1 ? 0 : f / PSIZE, fp = NP == 1 ? f : f % PSIZE;
        r = prow(fp / PW);
        const int cl = fp % PW;
        col = p * PW + 4 * ((cl >> 2) ^ swz(r)) + (cl & 3);
    }

    // This lane's share of every copy of the tile, fixed for the whole K loop: per copy
    // instruction, the byte offset of its data from the tile origin (row stride ld floats).
    // With EDGE, data beyond `mn` rows (KCONTIG) or columns (otherwise) along m or n gets an
    // offset past the buffer's range here; the k direction is checked per K-tile.
    struct Lane {
        unsigned off[CH];
    };
    template <bool EDGE>
    __host__ __device__ __forceinline__ static Lane plan(int64_t ld, int mn, int tid)
    {
        Lane L;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            int r, col;
            where(c, tid, r, col);
            L.off[c] = static_cast<unsigned>(((int64_t)r * ld + col) * 4);
            if (EDGE && !((KCONTIG ? r : col) < mn))
                L.off[c] = 0x80000000u;                 // past num_records: reads as zeros
        }
        return L;
    }

    // Queue this thread's copies of the tile whose origin is src into lds; `k` is how many
    // of the tile's k indices lie inside the matrix (EDGE only; only a K-tile that ends
    // past K needs the per-lane check). The buffer resource (one per tile, wave-uniform)
    // and the LDS destinations are the only per-step address work. With U, ld (row
    // stride) and mn (rows or columns inside the matrix along m or n) serve the 4-byte
    // copies of the K-tile that holds the end of K.
    template <bool EDGE>
    __device__ __forceinline__ static void load(const Lane &L, const float *src, int k, float *lds, int tid,
                                                int64_t ld = 0, int mn = 0)
    {
        if constexpr (U) {
            if (k <= KEXT) {
                words(src, ld, mn, k, lds, tid);
                return;
            }
        }
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS base in M0
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), 0, 0x7fffffff, 0x00020000);
        const bool partial = EDGE && k < KEXT;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            unsigned off = L.off[c];
            if (partial) {
                int r, col;
                where(c, tid, r, col);
                if (!((KCONTIG ? col : r) < k))
                    off = 0x80000000u;
            }
            lds_void *dst = (lds_void *)(lds + VW * (wave * 64 + c * NT));
            if constexpr (VW == 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, off, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, off, 0, 0, 0);
        }
    }

    // The same tile in the layout of 4-byte copies (the same LDS positions, copied a float
    // per lane).
    using Words = TileDMA<TR, TC, NT, KCONTIG, 1, Q16, PW>;

    // The whole tile in 4-byte copies, every float checked against mn (m or n) and k; the
    // offsets are computed copy by copy in a loop unrolled only by four, so this once-per-tile
    // path holds few registers (fully unrolled, the 256 x 256 tile spilled).
    __device__ __forceinline__ static void words(const float *src, int64_t ld, int mn, int k, float *lds, int tid)
    {
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), 0, 0x7fffffff, 0x00020000);
#pragma unroll 4
        for (int c = 0; c < Words::CH; ++c) {
            int r, col;
            Words::where(c, tid, r, col);
            const bool in = (KCONTIG ? r : col) < mn && (KCONTIG ? col : r) < k;
            const unsigned off = in ? static_cast<unsigned>(((int64_t)r * ld + col) * 4) : 0x80000000u;
            lds_void *dst = (lds_void *)(lds + wave * 64 + c * NT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, off, 0, 0, 0);
        }
    }
};

// Wait until at most n vector-memory operations of this wave are outstanding (the
// LDS copies above count as such); the other counters are left alone.
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier of the direct-copy pipeline: this wave's LDS reads have finished
// and at most n of its LDS copies are still in flight, then all waves meet. The
// __syncthreads() fence would also wait for every copy in flight (it counts them as
// LDS stores), which would leave no tile in flight across the barrier; the empty asm
// statements keep the compiler from moving memory accesses across it instead, and the
// scheduling barriers keep the matrix instructions on their side of it.
template <int n>
__device__ __forceinline__ void copy_barrier()
{
    static_assert(n >= 0 && n < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));  // vmcnt(n) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// W consecutive floats from LDS (W = 1, 2 or 4) as one 32-, 64- or 128-bit read.
template <int W>
__device__ __forceinline__ void lds_read(const float *p, float (&out)[W])
{
    if constexpr (W == 4) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(p);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (W == 2) {
        const floatx2 v = *reinterpret_cast<const floatx2 *>(p);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = p[0];
    }
}

// The two fp32 matrix instructions, as blocks of MB x MB outputs. Lane l supplies
// A(l % MB, l / MB) and B(l / MB, l % MB) and holds NACC accumulators; LG = 64 / MB lane
// groups each supply one k, so one instruction adds the outer products of LG k values.
//  - MB = 32: v_mfma_f32_32x32x2_f32, 16 accumulators, accumulator e of lane l is
//    D(8*(e/4) + 4*(l/32) + e%4, l%32).
//  - MB = 16: v_mfma_f32_16x16x4_f32, 4 accumulators, accumulator e of lane l is
//    D(4*(l/16) + e, l%16).
// Both are D(LG*4*(e/4) + 4*(l/MB) + e%4, l%MB). Each does MB*MB*LG multiply-adds per issue
// at the same rate per cycle, so the 16 x 16 form trades twice the issues for blocks a
// quarter of the size: finer tiles for small, skinny and ragged products.
template <int MB>
struct MfmaBlock;
template <>
struct MfmaBlock<32> {
    typedef floatx16 acc_t;
    static constexpr int NACC = 16, LG = 2;
    __device__ __forceinline__ static acc_t mma(float a, float b, const acc_t &c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};
template <>
struct MfmaBlock<16> {
    typedef floatx4 acc_t;
    static constexpr int NACC = 4, LG = 4;
    __device__ __forceinline__ static acc_t mma(float a, float b, const acc_t &c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------------
// MFMA kernel.
//
// Template parameters: BM x BN workgroup tile, BK k-depth per LDS stage, WGM x WGN
// waves over the tile, WGK wave groups along k, TA / TB whether op(A) / op(B) is a
// transpose, MB the matrix instruction's block (32 or 16). With WGK > 1 every wave group multiplies its own BK/WGK slice of each
// stage into its own accumulators, and at the end the groups add their accumulators
// through LDS in a fixed order (group 0 + 1 + 2 ...), so results stay reproducible;
// this puts more waves on each CU when the problem has few tiles, without any memory
// outside the workgroup. VEC selects 128-bit global loads/stores (operands 16-byte
// aligned, leading dimensions and contiguous extents multiples of 4); EDGE enables
// the bounds checks needed when M, N or K is not a multiple of the tile. Without VEC
// every element is checked.
//
// Each operand tile is staged in LDS in its memory layout (TileIO, padded rows): A as
// [BM][BK] (k contiguous), or [BK][BM] when transposed (m contiguous); B as [BK][BN] (n
// contiguous), or [BN][BK] when transposed (k contiguous).
//
// Lane layout: MfmaBlock above (for 32x32 blocks lane l supplies A(l%32, l/32) and
// B(l/32, l%32)). Remappings make every LDS read wide:
//  - k: within each group of KGRP = 4*LG k values (8 for 32x32 blocks, 16 for 16x16), lane
//    group h = l/MB takes k = 4h + s on matrix step s (s = 0..3). A and B use the same
//    map, so each issue still adds A(:,k)B(k,:) for LG distinct k and the 4 steps cover
//    all KGRP. An operand stored k-contiguous (A plain, B transposed) then gives lane l
//    its four values as one 128-bit read.
//  - m / n: an operand stored m- or n-contiguous (A transposed, B plain) has the
//    wave's blocks along that dimension interleaved, block b index c <-> wave index
//    c*T + b (T blocks), so lane l reads T consecutive values for one k in one read,
//    and for B writes T consecutive columns of C. For plain B with T = 3 or 6 (wave
//    tiles 48 or 96 wide) the blocks stay side by side and each is read one float per
//    lane, from a B tile kept in 32- or 16-wide panels (TileDMA).
// ---------------------------------------------------------------------------------
// One BM x BN tile of op(A) op(B) on matrix cores: the operand loaders, the LDS ring and
// the MFMA loop over a range of K-tiles (product), and the C update (epilogue). The
// whole-tile kernel below runs product over all of K; the stream-K kernel runs it over
// the K-tile ranges its workgroup owns.
template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, bool TA, bool TB, bool VEC,
          bool EDGE, int MB = 32, bool GS = false>
struct MfmaTile {
    static_assert(PF == 1 || PF == 2, "K-tiles in flight ahead of the one being multiplied");
    // GS: general-stride operands (column strides incA, incB, incC), loaded float by float
    // through registers; A and B are then read as stored, whatever their strides.
    static_assert(!GS || (!DMA && !TA && !TB && !VEC && EDGE), "general strides: staged, checked loads");
    static_assert(MB == 32 || MB == 16, "32x32 or 16x16 matrix blocks");
    using BLK = MfmaBlock<MB>;
    using acc_t = typename BLK::acc_t;
    static constexpr int NACC = BLK::NACC;                  // accumulators per lane and block
    static constexpr int LG = BLK::LG;                      // lane groups, one k each per issue
    static constexpr int KGRP = 4 * LG;                     // k per group of 4 matrix steps
    static constexpr bool USE_DMA = DMA;                    // direct HBM -> LDS copies
    // Direct copies are 16 bytes wide; on rows only 4-byte aligned (!VEC) the K-tile that
    // holds the end of K is copied in 4-byte words (TileDMA's U form).
    static constexpr bool UCOPY = DMA && !VEC;
    static constexpr int NT = WGM * WGN * WGK * 64;
    static constexpr int KSLICE = BK / WGK;                    // k per stage handled by one wave group
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;       // wave tile
    static constexpr int TM = WTM / MB, TN = WTN / MB;         // blocks per wave
    // B's blocks side by side in the wave tile (lane column li of block b is wave column
    // b*MB + li): always for transposed B, and for plain B when a lane's TN columns cannot
    // be one 1-, 2- or 4-float read (TN = 3 or 6); otherwise they are interleaved.
    static constexpr bool BSIDE = TB || !(TN == 1 || TN == 2 || TN == 4);
    // Panel width of a plain B tile in LDS: rows of 3 * 2^j floats are split into 32- or
    // 16-wide panels (TileDMA), which the side-by-side blocks read one panel at a time.
    static constexpr int BPW = (TB || BN % 64 == 0 || BN == 16 || BN == 32) ? (TB ? BK : BN) : (BN % 32 == 0 ? 32 : 16);
    using AIO = typename std::conditional<USE_DMA,
                                          TileDMA<TA ? BK : BM, TA ? BM : BK, NT, !TA, 4, MB == 16 && TM == 1,
                                                  TA ? BM : BK, UCOPY>,
                                          TileIO<TA ? BK : BM, TA ? BM : BK, NT>>::type;
    using BIO = typename std::conditional<USE_DMA,
                                          TileDMA<TB ? BN : BK, TB ? BK : BN, NT, TB, 4, MB == 16 && (TN == 1 || BSIDE),
                                                  BPW, UCOPY>,
                                          TileIO<TB ? BN : BK, TB ? BK : BN, NT>>::type;
    static constexpr int STAGE = AIO::SIZE + BIO::SIZE;
    static constexpr int NSTAGE = USE_DMA ? PF + 1 : 2;     // LDS stages in the ring
    static_assert(WTM % MB == 0 && WTN % MB == 0, "wave tile must be whole blocks");
    static_assert(!TA || TM == 1 || TM == 2 || TM == 4, "interleaved m blocks read 1, 2 or 4 floats");
    static_assert(BK % (KGRP * WGK) == 0, "each wave group consumes k in whole groups");
    static constexpr int RED = (WGK - 1) * BM * BN;         // partial sums of groups 1..WGK-1
    static constexpr int SMEM = NSTAGE * STAGE > RED ? NSTAGE * STAGE : RED;
    // Waves per SIMD the register budget is sized for: one for waves holding 256 or more
    // accumulators (the wave gets the whole 512-register file), else at least two, so that
    // two 256-thread workgroups fit on a CU.
    static constexpr int WPE = TM * TN * NACC >= 256 ? 1 : (NT >= 512 ? NT / 256 : 2);
    // Double-buffered fragment reads (next group's reads in flight while this group is
    // multiplied). Measured on MI355X: a gain for the direct-copy loop, for one K-tile
    // in flight and for waves holding a single 32x32 block; with two K-tiles in flight and
    // larger wave tiles the extra registers cost more than the overlap gains (the 256x256
    // kernel would spill), so those keep single fragments read next to their use unless
    // the wave has the whole register file.
    static constexpr bool FRAG = USE_DMA || PF == 1 || TM * TN == 1 || WPE == 1;
    static_assert(SMEM * 4 <= 160 * 1024, "LDS exceeds 160 KiB");

    // Multiply K-tiles [kt0, kt1) of the tile at (m0, n0) into acc, which starts at zero;
    // tid_in is the thread's index in the workgroup. With WGK > 1 the groups' sums end up
    // in the waves of group 0; the other waves return false and hold nothing.
    template <class Args>
    __device__ __forceinline__ static bool product(const Args &p, float *smem, int m0, int n0, int kt0,
                                                   int kt1, acc_t (&acc)[TM][TN], int tid_in)
    {
        const int M = p.M, N = p.N, K = p.K;
        const float *__restrict__ A = p.A + (int64_t)blockIdx.z * p.strideA;
        const float *__restrict__ B = p.B + (int64_t)blockIdx.z * p.strideB;
        const int64_t lda = p.lda, ldb = p.ldb;
        const int kbase = kt0 * BK;                         // first k of the range

        const int tid = tid_in;
        const int lane = tid & 63, wave = tid >> 6;
        const int wk = wave / (WGM * WGN);
        const int wm = (wave % (WGM * WGN)) / WGN, wn = wave % WGN;
        const int li = lane % MB, lg = lane / MB;   // row / column in the block, lane group

        // PF sets of staging registers: with PF = 2 a K-tile's global loads are issued two
        // stages before it is multiplied. `slot` is always a compile-time constant after
        // inlining, so the sets stay in registers.
        floatx4 ra[USE_DMA ? 1 : PF][AIO::CH], rb[USE_DMA ? 1 : PF][BIO::CH];

        // Global -> registers set `slot` for the K-tile starting kr after the range's first k
        // (zero outside the matrix).
        auto load_tile = [&](int kr, int slot) __attribute__((always_inline)) {
            if constexpr (GS) {
                const int k0 = kbase + kr;
                AIO::template load<false, true, true>(ra[slot], A + (int64_t)m0 * lda + (int64_t)k0 * p.incA, lda,
                                                      M - m0, K - k0, tid, p.incA);
                BIO::template load<false, true, true>(rb[slot], B + (int64_t)k0 * ldb + (int64_t)n0 * p.incB, ldb,
                                                      K - k0, N - n0, tid, p.incB);
            } else if constexpr (!USE_DMA) {
                const int k0 = kbase + kr;
                if constexpr (TA)
                    AIO::template load<VEC, EDGE>(ra[slot], A + (int64_t)k0 * lda + m0, lda, K - k0, M - m0, tid);
                else
                    AIO::template load<VEC, EDGE>(ra[slot], A + (int64_t)m0 * lda + k0, lda, M - m0, K - k0, tid);
                if constexpr (TB)
                    BIO::template load<VEC, EDGE>(rb[slot], B + (int64_t)n0 * ldb + k0, ldb, N - n0, K - k0, tid);
                else
                    BIO::template load<VEC, EDGE>(rb[slot], B + (int64_t)k0 * ldb + n0, ldb, K - k0, N - n0, tid);
            }
        };

        // Registers set `slot` -> LDS stage `st`.
        auto store_tile = [&](int st, int slot) __attribute__((always_inline)) {
            if constexpr (!USE_DMA) {
                float *As = smem + st * STAGE;
                AIO::store(ra[slot], As, tid);
                BIO::store(rb[slot], As + AIO::SIZE, tid);
            }
        };

        // Direct copies of the K-tile starting kr after the range's first k into LDS stage `st`
        // (DMA path). Each lane's offsets inside a tile are the same for every K-tile.
        const typename AIO::Lane a_lane = AIO::template plan<EDGE>(lda, M - m0, tid);
        const typename BIO::Lane b_lane = BIO::template plan<EDGE>(ldb, N - n0, tid);
        auto copy_tile = [&](int kr, int st) __attribute__((always_inline)) {
            if constexpr (USE_DMA) {
                const int k0 = kbase + kr;
                float *As = smem + st * STAGE;
                if constexpr (TA)
                    AIO::template load<EDGE>(a_lane, A + (int64_t)k0 * lda + m0, K - k0, As, tid, lda, M - m0);
                else
                    AIO::template load<EDGE>(a_lane, A + (int64_t)m0 * lda + k0, K - k0, As, tid, lda, M - m0);
                if constexpr (TB)
                    BIO::template load<EDGE>(b_lane, B + (int64_t)n0 * ldb + k0, K - k0, As + AIO::SIZE, tid, ldb,
                                             N - n0);
                else
                    BIO::template load<EDGE>(b_lane, B + (int64_t)k0 * ldb + n0, K - k0, As + AIO::SIZE, tid, ldb,
                                             N - n0);
            }
        };

    #pragma unroll
        for (int a = 0; a < TM; ++a)
    #pragma unroll
            for (int b = 0; b < TN; ++b)
    #pragma unroll
                for (int e = 0; e < NACC; ++e)
                    acc[a][b][e] = 0.f;

        // This lane's first row of A / column of B inside the tile: plain A rows are
        // a*MB + li (blocks side by side), transposed A rows li*TM + a (interleaved);
        // B columns likewise, side by side or interleaved (BSIDE).
        const int a_idx = wm * WTM + (TA ? li * TM : li);
        const int b_idx = wn * WTN + (BSIDE ? li : li * TN);

        // One stage: KSLICE/KGRP groups of KGRP k values, 4 matrix steps each.
        auto compute = [&](int st) __attribute__((always_inline)) {
            const float *As = smem + st * STAGE;
            const float *Bs = As + AIO::SIZE;
    #pragma unroll
            for (int kk = 0; kk < KSLICE; kk += KGRP) {
                const int kg = wk * KSLICE + kk;
                floatx4 af[TA ? 1 : TM], bf[TB ? TN : 1];
                if constexpr (!TA) {
    #pragma unroll
                    for (int a = 0; a < TM; ++a)
                        af[a] = *reinterpret_cast<const floatx4 *>(&As[AIO::elem(a_idx + a * MB, kg + 4 * lg)]);
                }
                if constexpr (TB) {
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
                        bf[b] = *reinterpret_cast<const floatx4 *>(&Bs[BIO::elem(b_idx + b * MB, kg + 4 * lg)]);
                }
    #pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int k = kg + 4 * lg + s;
                    float av[TM], bv[TN];
                    if constexpr (TA) {
                        lds_read<TM>(&As[AIO::elem(k, a_idx)], av);
                    } else {
    #pragma unroll
                        for (int a = 0; a < TM; ++a)
                            av[a] = af[a][s];
                    }
                    if constexpr (TB) {
    #pragma unroll
                        for (int b = 0; b < TN; ++b)
                            bv[b] = bf[b][s];
                    } else if constexpr (BSIDE) {
    #pragma unroll
                        for (int b = 0; b < TN; ++b)
                            bv[b] = Bs[BIO::elem(k, b_idx + b * MB)];
                    } else {
                        lds_read<TN>(&Bs[BIO::elem(k, b_idx)], bv);
                    }
    #pragma unroll
                    for (int a = 0; a < TM; ++a)
    #pragma unroll
                        for (int b = 0; b < TN; ++b)
                            acc[a][b] = BLK::mma(av[a], bv[b], acc[a][b]);
                }
            }
        };

        // Fragment form (FRAG): the A and B values of one group of KGRP k (4 per lane) for
        // every block, read from LDS in one batch, so the reads of the next group can be in
        // flight while this one is multiplied.
        constexpr int NG = KSLICE / KGRP;                   // groups of k per stage and wave group
        float fa[FRAG ? 2 : 1][4][TM], fb[FRAG ? 2 : 1][4][TN];
        auto read_frag = [&](int st, int g, int buf) __attribute__((always_inline)) {
            const float *As = smem + st * STAGE;
            const float *Bs = As + AIO::SIZE;
            const int kg = wk * KSLICE + KGRP * g + 4 * lg;
            if constexpr (TA) {
    #pragma unroll
                for (int s = 0; s < 4; ++s)
                    lds_read<TM>(&As[AIO::elem(kg + s, a_idx)], fa[buf][s]);
            } else {
    #pragma unroll
                for (int a = 0; a < TM; ++a) {
                    const floatx4 v = *reinterpret_cast<const floatx4 *>(&As[AIO::elem(a_idx + a * MB, kg)]);
    #pragma unroll
                    for (int s = 0; s < 4; ++s)
                        fa[buf][s][a] = v[s];
                }
            }
            if constexpr (TB) {
    #pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const floatx4 v = *reinterpret_cast<const floatx4 *>(&Bs[BIO::elem(b_idx + b * MB, kg)]);
    #pragma unroll
                    for (int s = 0; s < 4; ++s)
                        fb[buf][s][b] = v[s];
                }
            } else if constexpr (BSIDE) {
    #pragma unroll
                for (int s = 0; s < 4; ++s)
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
                        fb[buf][s][b] = Bs[BIO::elem(kg + s, b_idx + b * MB)];
            } else {
    #pragma unroll
                for (int s = 0; s < 4; ++s)
                    lds_read<TN>(&Bs[BIO::elem(kg + s, b_idx)], fb[buf][s]);
            }
        };
        auto mma_frag = [&](int buf) __attribute__((always_inline)) {
    #pragma unroll
            for (int s = 0; s < 4; ++s)
    #pragma unroll
                for (int a = 0; a < TM; ++a)
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
                        acc[a][b] = BLK::mma(fa[buf][s][a], fb[buf][s][b], acc[a][b]);
        };

        // Pipeline over the range's nk K-tiles, one barrier per K-tile.
        const int nk = kt1 - kt0;
        if constexpr (USE_DMA) {
            // PF + 1 LDS stages. Step t queues the copies of tile t+PF into stage (t+PF) %
            // NSTAGE (read last during step t-1, so free after that step's barrier),
            // multiplies stage t % NSTAGE, waits until its own copies of tile t+1 have landed
            // (the PF-1 newer tiles may stay in flight) and meets the others at the barrier.
            // Past the end the last tile is copied again, so the count of copies in flight
            // is the same on every step. (In the U form the K-tile holding the end of K takes
            // four times the copies; it is the last tile, or a repeat of it, so the waits
            // below, counted for 16-byte tiles, then only wait for more than they need.)
            // Inside a step, group g+1's fragments are read while group g is multiplied; the
            // last group is multiplied after the barrier, while group 0 of the next stage
            // is read (past the last step that read is of a stage nobody uses; harmless).
            constexpr int COPIES = AIO::CH + BIO::CH;       // copy instructions per thread per tile
    #pragma unroll
            for (int q = 0; q < PF; ++q)
                copy_tile((q < nk ? q : nk - 1) * BK, q);
            wait_vmcnt<0>();
            __syncthreads();
            read_frag(0, 0, 0);
            if constexpr (NG % 2 == 0) {
                // Every stage starts with its group 0 in buffer 0.
                for (int t = 0; t < nk; ++t) {
                    const int ahead = t + PF < nk ? t + PF : nk - 1;
                    copy_tile(ahead * BK, (t + PF) % NSTAGE);
                    const int st = t % NSTAGE;
    #pragma unroll
                    for (int g = 0; g + 1 < NG; ++g) {
                        read_frag(st, g + 1, (g + 1) & 1);
                        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
                        mma_frag(g & 1);
                    }
                    copy_barrier<(PF - 1) * COPIES>();
                    read_frag((t + 1) % NSTAGE, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_frag(1);
                }
            } else {
                // An odd number of groups per stage: a step whose group 0 sits in buffer P
                // leaves the next step's group 0 in buffer 1 - P, so the steps alternate P = 0, 1
                // (unrolled by two to keep the buffer indices compile-time constants). The loop
                // for even counts stays a form of its own: with both folded into this one, the
                // 64 x 64 x 64 four-wave-row kernel ran 30% slower on 1536 x 2048 x 2048 (97 to
                // 126 us) with fewer workgroups resident, though its machine code differed in
                // a handful of scalar instructions only; the cause was not found.
                auto step = [&](int t, auto parity) __attribute__((always_inline)) {
                    constexpr int P = decltype(parity)::value;
                    const int ahead = t + PF < nk ? t + PF : nk - 1;
                    copy_tile(ahead * BK, (t + PF) % NSTAGE);
                    const int st = t % NSTAGE;
    #pragma unroll
                    for (int g = 0; g + 1 < NG; ++g) {
                        read_frag(st, g + 1, (g + 1 + P) & 1);
                        __builtin_amdgcn_sched_barrier(0);
                        mma_frag((g + P) & 1);
                    }
                    copy_barrier<(PF - 1) * COPIES>();
                    read_frag((t + 1) % NSTAGE, 0, 1 - P);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_frag((NG - 1 + P) & 1);
                };
                int t = 0;
                for (; t + 1 < nk; t += 2) {
                    step(t, std::integral_constant<int, 0>{});
                    step(t + 1, std::integral_constant<int, 1>{});
                }
                if (t < nk)
                    step(t, std::integral_constant<int, 0>{});
            }
            wait_vmcnt<0>();    // no copy may still write LDS once it is reused or released
        } else if constexpr (PF == 1) {
            static_assert(NG % 2 == 0, "fragment buffers alternate within a stage");
            load_tile(0, 0);
            store_tile(0, 0);
            __syncthreads();
            read_frag(0, 0, 0);
            for (int t = 0; t + 1 < nk; ++t) {
                load_tile((t + 1) * BK, 0);  // in flight while this stage is multiplied
#pragma unroll
                for (int g = 0; g + 1 < NG; ++g) {
                    read_frag(t & 1, g + 1, (g + 1) & 1);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_frag(g & 1);
                }
                store_tile((t + 1) & 1, 0);  // other stage: its last reader finished before the previous barrier
                __syncthreads();
                read_frag((t + 1) & 1, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                mma_frag(1);
            }
#pragma unroll
            for (int g = 0; g + 1 < NG; ++g) {
                read_frag((nk - 1) & 1, g + 1, (g + 1) & 1);
                __builtin_amdgcn_sched_barrier(0);
                mma_frag(g & 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_frag(1);
        } else {
            // Entering step t: stage t%2 holds K-tile t, register set (t+1)%2 holds tile t+1
            // (loaded during step t-1) and set t%2 is free. Step t loads tile t+2 into set
            // t%2 (the last tile again once past the end, so the load needs no condition),
            // multiplies stage t%2, then stores set (t+1)%2 into stage (t+1)%2.
            // With FRAG, fragments are double-buffered as in the direct-copy loop: group g+1's
            // reads are in flight while group g is multiplied, and the next stage's first group
            // is read right after the barrier, while this stage's last group is multiplied.
            static_assert(!FRAG || NG % 2 == 0, "fragment buffers alternate within a stage");
            auto groups = [&](int st) __attribute__((always_inline)) {
                if constexpr (FRAG) {
#pragma unroll
                    for (int g = 0; g + 1 < NG; ++g) {
                        read_frag(st, g + 1, (g + 1) & 1);
                        __builtin_amdgcn_sched_barrier(0);
                        mma_frag(g & 1);
                    }
                } else {
                    compute(st);
                }
            };
            auto step = [&](int t, int s) __attribute__((always_inline)) {
                const int ahead = t + 2 < nk ? t + 2 : nk - 1;
                load_tile(ahead * BK, s);
                groups(s);
                store_tile(1 - s, 1 - s);
                __syncthreads();
                if constexpr (FRAG) {
                    read_frag(1 - s, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_frag(1);
                }
            };
            load_tile(0, 0);
            load_tile((nk > 1 ? 1 : 0) * BK, 1);
            store_tile(0, 0);
            __syncthreads();
            if constexpr (FRAG)
                read_frag(0, 0, 0);
            int t = 0;
            for (; t + 2 < nk; t += 2) {     // steps t and t+1, both before the last tile
                step(t, 0);
                step(t + 1, 1);
            }
            if (t + 1 < nk) {
                step(t, 0);
                ++t;
            }
            groups((nk - 1) & 1);            // the last tile: no next stage to read
            if constexpr (FRAG) {
                __builtin_amdgcn_sched_barrier(0);
                mma_frag(1);
            }
        }

        if constexpr (WGK > 1) {
            // Groups 1..WGK-1 hand their partial sums to group 0 through LDS (the ring is
            // free once every wave has passed the barrier); group 0 adds them in group order.
            constexpr int PER_WAVE = TM * TN * NACC * 64;
            const int slot = wm * WGN + wn;
            __syncthreads();
            if (wk > 0) {
                float *dst = smem + ((wk - 1) * (WGM * WGN) + slot) * PER_WAVE;
    #pragma unroll
                for (int a = 0; a < TM; ++a)
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
    #pragma unroll
                        for (int e = 0; e < NACC; ++e)
                            dst[((a * TN + b) * NACC + e) * 64 + lane] = acc[a][b][e];
            }
            __syncthreads();
            if (wk > 0)
                return false;
    #pragma unroll
            for (int g = 1; g < WGK; ++g) {
                const float *src = smem + ((g - 1) * (WGM * WGN) + slot) * PER_WAVE;
    #pragma unroll
                for (int a = 0; a < TM; ++a)
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
    #pragma unroll
                        for (int e = 0; e < NACC; ++e)
                            acc[a][b][e] += src[((a * TN + b) * NACC + e) * 64 + lane];
            }
        }
        return true;
    }

    template <class Args>
    __device__ __forceinline__ static void epilogue(const Args &p, int m0, int n0,
                                                    const acc_t (&acc)[TM][TN], int tid_in)
    {
        const int M = p.M, N = p.N;
        float *__restrict__ C = p.C + (int64_t)blockIdx.z * p.strideC;
        const int64_t ldc = p.ldc;
        const int tid = tid_in;
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = (wave % (WGM * WGN)) / WGN, wn = wave % WGN;
        const int li = lane % MB, lg = lane / MB;
        const int b_idx = wn * WTN + (BSIDE ? li : li * TN);
        // Epilogue: C = act(alpha*acc + beta*C + bias), C unread when beta == 0. One block
        // row at a time: all of the block's reads of C are issued before the first is used,
        // so the block waits out one memory round trip (two with EB = 8) rather than one per
        // entry. C is written with non-temporal stores: this kernel never reads it back, and
        // streamed out it leaves the L2 to the operand panels other tiles still read (back to
        // back 2-5% faster on the GPT-2 layers and attention's scores, the same at 4096^3, 1%
        // slower on the ragged 1000 x 1537 x 777). Lane columns: TN consecutive ones
        // (interleaved blocks), or one per MB-column block (side by side). Rows: those of
        // accumulator element e, see MfmaBlock.
        const float alpha = p.alpha, beta = p.beta;
        const float *bias = p.bias;
        const int act = p.act;
        int64_t incc = 1;                                   // column stride of C
        if constexpr (GS)
            incc = p.incC;
        const bool read_c = beta != 0.f, has_bias = bias != nullptr;
        const bool full = !EDGE || (m0 + BM <= M && n0 + BN <= N);   // whole tile inside C
        // 128- or 64-bit accesses of a lane's TN consecutive columns: aligned, and (N % 4 == 0,
        // first column a multiple of TN) the group is either wholly inside C or wholly out.
        constexpr bool VCOL = VEC && !BSIDE && (TN == 2 || TN == 4);
        int gc[TN];
    #pragma unroll
        for (int b = 0; b < TN; ++b)
            gc[b] = n0 + b_idx + (BSIDE ? MB * b : b);
        float bj[TN];
    #pragma unroll
        for (int b = 0; b < TN; ++b)
            bj[b] = (has_bias && (full || gc[b] < N)) ? bias[gc[b]] : 0.f;
        auto row_of = [&](int a, int e) __attribute__((always_inline)) {
            const int r = 4 * LG * (e / 4) + 4 * lg + (e % 4);      // row inside the block
            return m0 + wm * WTM + (TA ? r * TM + a : a * MB + r);
        };
        // Entries per batch of reads: the whole block (16 or 4), or 8 where four waves share
        // a SIMD and each has only 128 registers.
        constexpr int EB = NT >= 1024 && NACC > 8 ? 8 : NACC;
    #pragma unroll
        for (int a = 0; a < TM; ++a)
    #pragma unroll
        for (int e0 = 0; e0 < NACC; e0 += EB) {
            float cv[NACC][TN];
            if (read_c) {
    #pragma unroll
                for (int e = e0; e < e0 + EB; ++e) {
                    const int gr = row_of(a, e);
                    const float *crow = C + (int64_t)gr * ldc;
                    if constexpr (VCOL) {
                        using vec_t = typename std::conditional<TN == 4, floatx4, floatx2>::type;
                        vec_t v{};
                        if (full || (gr < M && gc[0] < N))
                            v = *reinterpret_cast<const vec_t *>(crow + gc[0]);
    #pragma unroll
                        for (int b = 0; b < TN; ++b)
                            cv[e][b] = v[b];
                    } else {
    #pragma unroll
                        for (int b = 0; b < TN; ++b)
                            cv[e][b] = (full || (gr < M && gc[b] < N)) ? crow[gc[b] * incc] : 0.f;
                    }
                }
            }
    #pragma unroll
            for (int e = e0; e < e0 + EB; ++e) {
                const int gr = row_of(a, e);
                float *crow = C + (int64_t)gr * ldc;
                float out[TN];
    #pragma unroll
                for (int b = 0; b < TN; ++b)
                    out[b] = finish_value(acc[a][b][e], alpha, beta, read_c ? cv[e][b] : 0.f, has_bias, bj[b], act);
                if constexpr (VCOL) {
                    using vec_t = typename std::conditional<TN == 4, floatx4, floatx2>::type;
                    vec_t v;
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
                        v[b] = out[b];
                    if (full || (gr < M && gc[0] < N))
                        __builtin_nontemporal_store(v, reinterpret_cast<vec_t *>(crow + gc[0]));
                } else {
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
                        if (full || (gr < M && gc[b] < N))
                            __builtin_nontemporal_store(out[b], &crow[gc[b] * incc]);
                }
            }
        }
    }
};

// Fringe columns: the last r = p.fringe columns of C (1 <= r <= kFringeCols), which the
// tile grid leaves out when it stops at the last whole column of tiles. One workgroup takes
// kFringeRows rows of C; its waves and lanes split K (thread t of wave w takes k = 64 (w + W u)
// + lane, u = 0, 1, ...) and each thread sums, for those rows, the products with the last R
// columns of B, R a compile-time 1, 2, 4 or 8 >= r (N >= R always, since the grid holds a
// whole column of tiles). The R floats of a row of B come in one or two vector loads that the
// rows share (and the rows of A in one, when A is transposed), so a step issues a few loads
// rather than one per entry: one per entry, each lane on its own row of B, runs at the rate
// the cache takes line requests, not at its bandwidth. Indices past K or M are clamped, so
// every load is unconditional, and the products of clamped k are dropped. Then a butterfly of
// lane exchanges adds the G R sums over the wave, halving them at each step (G R - 1 exchanges
// for G R <= 16 sums rather than 6 G R), and the waves' totals meet in LDS.
constexpr int kFringeCols = 8;
constexpr int kFringeRows = 2;

typedef float floatx2u __attribute__((ext_vector_type(2), aligned(4)));

template <int NT, bool TA, bool TB, int R>
__device__ __forceinline__ void fringe_columns(const GemmArgs &p, int f, float *red, int tid)
{
    constexpr int G = kFringeRows, W = NT / 64, NV = G * R;
    constexpr int LOGN = NV == 2 ? 1 : NV == 4 ? 2 : NV == 8 ? 3 : NV == 16 ? 4 : 5;
    static_assert(NV == (1 << LOGN), "G R must be a power of two up to 32");
    // Steps of 64 W k whose loads are in flight together: U (G + R) loaded floats, their
    // addresses and the G R sums stay under what the tile kernels hold, so the branch does
    // not lower the tiles' occupancy.
    constexpr int U = R <= 2 ? 4 : R == 4 ? 2 : 1;
    const int lane = tid & 63, w = tid >> 6;
    const int M = p.M, K = p.K, r = p.fringe, c0 = p.N - R;
    const int m0 = f * G;
    const bool full = m0 + G <= M;
    const float *__restrict__ A = p.A + (int64_t)blockIdx.z * p.strideA;
    const float *__restrict__ B = p.B + (int64_t)blockIdx.z * p.strideB;
    float *__restrict__ C = p.C + (int64_t)blockIdx.z * p.strideC;
    const int64_t lda = p.lda, ldb = p.ldb;
    // Rows of A (plain) and columns of B (transposed) are read from one base each with
    // 32-bit offsets (the host takes fringes only for row strides under 2^20 floats).
    const float *__restrict__ Am = A + (int64_t)m0 * lda;
    const float *__restrict__ Bn = B + (int64_t)c0 * ldb;
    int arow[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        arow[g] = (m0 + g < M ? g : M - 1 - m0) * (int)lda;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        v[i] = 0.f;
    for (int kb = 64 * w + lane; kb < K; kb += 64 * W * U) {
        float a[U][G], b[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + 64 * W * u;
            const int kc = k < K ? k : K - 1;
            if constexpr (TA) {
                const float *ak = A + (int64_t)kc * lda;
                if (full) {     // the G rows m0.. in one load of exactly G floats
                    static_assert(G == 2, "one two-float load per k");
                    const floatx2u x = *reinterpret_cast<const floatx2u *>(ak + m0);
                    a[u][0] = x[0];
                    a[u][1] = x[1];
                } else {
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        a[u][g] = ak[m0 + g < M ? m0 + g : M - 1];
                }
            } else {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    a[u][g] = Am[arow[g] + kc];
            }
            if constexpr (TB) {
#pragma unroll
                for (int j = 0; j < R; ++j)
                    b[u][j] = Bn[j * (int)ldb + kc];
            } else {
                const float *bk = B + (int64_t)kc * ldb + c0;
                if constexpr (R == 1) {
                    b[u][0] = bk[0];
                } else if constexpr (R == 2) {
                    const floatx2u x = *reinterpret_cast<const floatx2u *>(bk);
                    b[u][0] = x[0];
                    b[u][1] = x[1];
                } else {
#pragma unroll
                    for (int q = 0; q < R / 4; ++q) {
                        const floatx4u x = *reinterpret_cast<const floatx4u *>(bk + 4 * q);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            b[u][4 * q + e] = x[e];
                    }
                }
            }
            if (k >= K) {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    a[u][g] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int j = 0; j < R; ++j)
                    v[g * R + j] = fmaf(a[u][g], b[u][j], v[g * R + j]);
    }
    // Halving steps (offsets 32, 16, ...): the lane keeps the half of its sums picked by its
    // bit at that offset and adds its partner's copy of that half. After LOGN steps lane l
    // holds one sum, index l >> (6 - LOGN), over the 2^LOGN lanes that differ from l only in
    // the top LOGN bits; plain exchanges over the remaining offsets complete it over the wave.
#pragma unroll
    for (int st = 0; st < LOGN; ++st) {
        const int o = 32 >> st;
        const int half = NV >> (st + 1);
        const bool hi = (lane & o) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = hi ? v[i] : v[i + half];
            const float keep = hi ? v[i + half] : v[i];
            v[i] = keep + __shfl_xor(send, o);
        }
    }
#pragma unroll
    for (int o = 32 >> LOGN; o > 0; o >>= 1)
        v[0] += __shfl_xor(v[0], o);
    if ((lane & ((64 >> LOGN) - 1)) == 0)
        red[w * NV + (lane >> (6 - LOGN))] = v[0];
    __syncthreads();
    if (tid < NV) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < W; ++q)
            t += red[q * NV + tid];
        const int g = tid / R, j = tid % R;
        if (j >= R - r && m0 + g < M) {
            const int col = c0 + j;
            float *cptr = C + (int64_t)(m0 + g) * p.ldc + col;
            *cptr = finish(t, p.alpha, p.beta, cptr, p.bias, col, p.act);
        }
    }
}

// One workgroup per output tile. With p.fringe = r > 0 the tiles cover the first N - r
// columns (a whole number of tiles) and the workgroups after them compute the last r
// columns, kFringeRows rows each (fringe_columns): a thin strip of columns then costs a
// short pass rather than a column of nearly empty tiles.
template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, bool TA, bool TB, bool VEC,
          bool EDGE, int MB>
__global__ void __launch_bounds__(WGM * WGN * WGK * 64)
__attribute__((amdgpu_waves_per_eu(MfmaTile<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, VEC, EDGE, MB>::WPE)))
sgemm_mfma(GemmArgs p, int group_m)
{
    using T = MfmaTile<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, VEC, EDGE, MB>;
    constexpr int NT = WGM * WGN * WGK * 64;
    __shared__ __attribute__((aligned(16))) float smem[T::SMEM];
    const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N - p.fringe, BN);
    static_assert(T::SMEM >= NT / 64 * kFringeRows * kFringeCols, "LDS too small for the fringe sums");
    if (p.fringe > 0 && (int)blockIdx.x >= tiles_m * tiles_n) {
        const int f = blockIdx.x - tiles_m * tiles_n;
        if (p.fringe <= 1)
            fringe_columns<NT, TA, TB, 1>(p, f, smem, threadIdx.x);
        else if (p.fringe <= 2)
            fringe_columns<NT, TA, TB, 2>(p, f, smem, threadIdx.x);
        else if (p.fringe <= 4)
            fringe_columns<NT, TA, TB, 4>(p, f, smem, threadIdx.x);
        else
            fringe_columns<NT, TA, TB, 8>(p, f, smem, threadIdx.x);
        return;
    }
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    typename T::acc_t acc[T::TM][T::TN];
    if (T::product(p, smem, tm * BM, tn * BN, 0, ceil_div(p.K, BK), acc, threadIdx.x))
        T::epilogue(p, tm * BM, tn * BN, acc, threadIdx.x);
}

// The same tile kernel on general-stride operands (any row and column strides of A, B
// and C, zero included for A and B): register-staged, element-wise, checked loads.
template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int MB>
__global__ void __launch_bounds__(WGM * WGN * WGK * 64)
__attribute__((amdgpu_waves_per_eu(MfmaTile<BM, BN, BK, WGM, WGN, WGK, 1, false, false, false, false, true, MB,
                                            true>::WPE)))
sgemm_mfma_strided(StridedArgs p, int group_m)
{
    using T = MfmaTile<BM, BN, BK, WGM, WGN, WGK, 1, false, false, false, false, true, MB, true>;
    __shared__ __attribute__((aligned(16))) float smem[T::SMEM];
    int tm, tn;
    tile_coords(blockIdx.x, ceil_div(p.M, BM), ceil_div(p.N, BN), group_m, tm, tn);
    typename T::acc_t acc[T::TM][T::TN];
    if (T::product(p, smem, tm * BM, tn * BN, 0, ceil_div(p.K, BK), acc, threadIdx.x))
        T::epilogue(p, tm * BM, tn * BN, acc, threadIdx.x);
}

// Work split of a stream-K launch (computed on the host).
struct StreamK {
    float *partials;        // 2 slots of BM*BN floats per sharing workgroup: its first and last tile
    unsigned *counters;     // one per tile; zero before the launch, left zero after it
    int tiles_m, tiles_n;
    int iters;              // K-tiles per output tile, I
    int group_m;
    int work;               // tiles * I, the K-tile steps of the whole product; (grid+1)*work < 2^31
    int dp;                 // leading tiles taken whole, one per workgroup (a multiple of 8); the
                            // other workgroups share the remaining steps
};

// Stream-K: the tiles * I K-tile steps of the product, taken in tile order, are split
// into contiguous ranges, one per workgroup, so every CU does the same amount of work
// whatever the tile count. The first sk.dp workgroups take one whole tile each (the
// first sk.dp tiles, as the data-parallel kernel would); the other G - dp workgroups
// split the remaining steps into equal ranges. Their count is at most the number of those
// steps, so no range is empty and the workgroups whose ranges meet a tile are exactly
// those between the owners of its first and last step. A workgroup walks its range tile
// by tile. A tile wholly inside the range gets the ordinary epilogue. A tile the range
// covers only in part leaves its partial sum in the workgroup's slot and takes a ticket
// from the tile's counter; the contributor that draws the last ticket adds the partial
// sums in contributor order (the same order whoever comes last, so results do not depend
// on timing) and writes C. No workgroup ever waits for another.
// Each part is spread over the XCDs on its own (dp is a multiple of their count, so a
// workgroup keeps its XCD), so the whole tiles and the shared ranges each land evenly on
// every XCD, and neighbouring ranges share an XCD's L2.
template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, bool TA, bool TB, bool VEC,
          bool EDGE, int MB>
__global__ void __launch_bounds__(WGM * WGN * WGK * 64)
sgemm_mfma_sk(GemmArgs p, StreamK sk)
{
    using T = MfmaTile<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, VEC, EDGE, MB>;
    constexpr int TILE = BM * BN;
    constexpr int NACC = T::NACC;
    constexpr int PER_WAVE = T::TM * T::TN * NACC * 64;   // one wave's accumulators
    __shared__ __attribute__((aligned(16))) float smem[T::SMEM];
    __shared__ unsigned ticket;

    const int G = gridDim.x;
    int I = sk.iters;
    const int b = blockIdx.x;
    int D = sk.dp;
    int WS = sk.work - D * I, GS = G - D;               // the shared steps and their workgroups
    const int g = b < D ? xcd_contiguous(b, D) : D + xcd_contiguous(b - D, GS);
    // The split's constants are kept in vector registers: they serve a few computations per
    // tile, and held as scalars across the K loop they pushed its scalar registers into spills
    // (re-reading them from the kernel's arguments instead made the loop 20% slower). Results
    // that steer control flow are made uniform again with readfirstlane.
    asm volatile("" : "+v"(D), "+v"(WS), "+v"(GS), "+v"(I));
    auto range_start = [&](int wg) {
        return __builtin_amdgcn_readfirstlane(wg <= D ? wg * I : D * I + (wg - D) * WS / GS);
    };
    auto owner = [&](int w) {                            // workgroup whose range holds step w
        return __builtin_amdgcn_readfirstlane(w < D * I ? w / I : D + ((w - D * I + 1) * GS - 1) / WS);
    };
    auto slot_of = [&](int wg, int t) { return t == range_start(wg) / I ? 0 : 1; };

    const int w_end = range_start(g + 1);
    for (int w = range_start(g); w < w_end;) {
        const int t = __builtin_amdgcn_readfirstlane(w / I);
        const int kt0 = __builtin_amdgcn_readfirstlane(w - t * I);
        const int kt1 = __builtin_amdgcn_readfirstlane((w_end - t * I) < I ? (w_end - t * I) : I);
        int tm, tn;
        band_coords(t, sk.tiles_m, sk.tiles_n, sk.group_m, tm, tn);
        typename T::acc_t acc[T::TM][T::TN];
        // The thread index passes through an empty asm statement on every tile, so the
        // per-lane addresses are recomputed per tile instead of being hoisted out of
        // this loop and held (with the accumulators) across the fixup and epilogue.
        int tid_l = threadIdx.x;
        asm volatile("" : "+v"(tid_l));
        const int lane = tid_l & 63, wslot = (tid_l >> 6) % (WGM * WGN);
        const bool holds = T::product(p, smem, tm * BM, tn * BN, kt0, kt1, acc, tid_l);
        bool finish = kt0 == 0 && kt1 == __builtin_amdgcn_readfirstlane(I);   // the whole tile is this workgroup's
        if (!finish) {
            const int first = owner(t * I), last = owner(t * I + I - 1);
            // Ordering of the hand-off. The accesses are relaxed, so the C++/HIP memory
            // model alone does not order them; the argument rests on how gfx950 executes
            // agent-scope accesses (the code sequences of the AMDGPU backend's memory model
            // for this target family):
            //  1. An agent-scope store is issued with sc1 and written through the XCD's L2
            //     to the device coherence point (memory side, shared by all XCDs). Stores
            //     count in vmcnt, and the counter drops only when the store is
            //     acknowledged there, so after wait_vmcnt<0>() every partial this wave
            //     stored is visible to an agent-scope access from any XCD.
            //  2. s_barrier (inside __syncthreads) makes thread 0's ticket RMW issue after
            //     every wave of the workgroup has passed step 1.
            //  3. The agent-scope fetch_add is atomic at the coherence point, so the
            //     counter's values are totally ordered; the contributor that reads
            //     last - first saw every other contributor's increment, each issued after
            //     that contributor's step 1.
            //  4. The winner's waves issue their partial loads after the barrier that
            //     follows the ticket's return. An agent-scope load (sc1) is served from the
            //     coherence point, never from a stale line in the XCD's L2, so it returns
            //     the stored partials.
            // A release/acquire pair (__threadfence, or release RMW + acquire load) would
            // make this follow from the language model, but on this target it is compiled
            // to buffer_wbl2 / buffer_inv of the whole XCD L2; with it the GPT-2 QKV layer
            // took 143 us instead of 41 us, so the per-access form is kept.
            if (holds) {
                float *dst = sk.partials + ((int64_t)(g - sk.dp) * 2 + slot_of(g, t)) * TILE + wslot * PER_WAVE;
#pragma unroll
                for (int a = 0; a < T::TM; ++a)
#pragma unroll
                    for (int b = 0; b < T::TN; ++b)
#pragma unroll
                        for (int e = 0; e < NACC; ++e)
                            __hip_atomic_store(&dst[((a * T::TN + b) * NACC + e) * 64 + lane], acc[a][b][e],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // Publish: this wave's stores are acknowledged, then every wave meets, then one
            // ticket is drawn.
            wait_vmcnt<0>();
            __syncthreads();
            if (tid_l == 0)
                ticket = __hip_atomic_fetch_add(&sk.counters[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            finish = ticket == (unsigned)(last - first);
            if (finish) {
                // Every contributor's partial, this workgroup's included, is in its slot: sum
                // them in contributor order straight into acc.
                for (int c = first; holds && c <= last; ++c) {
                    const float *src = sk.partials + ((int64_t)(c - sk.dp) * 2 + slot_of(c, t)) * TILE + wslot * PER_WAVE;
#pragma unroll
                    for (int a = 0; a < T::TM; ++a)
#pragma unroll
                        for (int b = 0; b < T::TN; ++b)
#pragma unroll
                            for (int e = 0; e < NACC; ++e) {
                                const float v = __hip_atomic_load(&src[((a * T::TN + b) * NACC + e) * 64 + lane],
                                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                acc[a][b][e] = c == first ? v : acc[a][b][e] + v;
                            }
                }
                if (tid_l == 0)                          // ready for the next launch
                    __hip_atomic_store(&sk.counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (finish && holds)
            T::epilogue(p, tm * BM, tn * BN, acc, tid_l);
        w = __builtin_amdgcn_readfirstlane((t + 1) * I);
        __syncthreads();                                 // the LDS ring is reused by the next tile
    }
}

}  // namespace sgemm_impl
