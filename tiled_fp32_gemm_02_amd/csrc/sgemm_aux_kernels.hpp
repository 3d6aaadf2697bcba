// The vector-ALU kernels of the library, included only by sgemm_api.hip:
//  - sgemm_tile16: the classic shared-memory kernel, one output per thread and 16x16
//    tiles (the GPT-2 post's hand-written matmul, "Tiled matrix multiplication"), kept
//    as the simplest correct rung and a baseline;
//  - sgemm_valu: the pages' register micro-tile on the vector ALU, 8x8 outputs per
//    thread updated by outer products, the reference that the matrix-core kernels are
//    measured against;
//  - sgemm_scale: C = act(beta*C + bias) for the quick returns (alpha == 0 or K == 0).
#pragma once

#include "sgemm_kernels.hpp"

namespace sgemm_impl {

// ---------------------------------------------------------------------------------
// Classic 16x16 shared-memory kernel: one output per thread. Each step stages one
// element of op(A) and one of op(B) per thread (zero outside the matrix), a barrier
// makes the tiles visible, 16 products are accumulated, and a second barrier keeps
// the next step's stores off tiles still being read. Grid: ceil(N/16) x ceil(M/16) x
// batch.
// ---------------------------------------------------------------------------------
template <bool TA, bool TB>
__global__ void __launch_bounds__(256) sgemm_tile16(GemmArgs p)
{
    __shared__ float sa[16][17];
    __shared__ float sb[16][17];
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
    const float *__restrict__ A = p.A + (int64_t)blockIdx.z * p.strideA;
    const float *__restrict__ B = p.B + (int64_t)blockIdx.z * p.strideB;
    float *__restrict__ C = p.C + (int64_t)blockIdx.z * p.strideC;
    float sum = 0.f;
    // K-tiles are counted rather than k advanced past K, and k offsets are compared with
    // what is left of K, so nothing overflows for K near 2^31.
    const int nk = ceil_div(p.K, 16);
    for (int t = 0; t < nk; ++t) {
        const int k0 = t * 16, kleft = p.K - k0;
        if (TA) {   // thread (ty, tx) stages op(A)(block row + tx, k0 + ty): reads run along m
            const int ar = blockIdx.y * 16 + tx;
            sa[tx][ty] = (ar < p.M && ty < kleft) ? A[(int64_t)(k0 + ty) * p.lda + ar] : 0.f;
        } else {
            sa[ty][tx] = (row < p.M && tx < kleft) ? A[(int64_t)row * p.lda + k0 + tx] : 0.f;
        }
        if (TB) {   // thread (ty, tx) stages op(B)(k0 + tx, block col + ty): reads run along k
            const int bc = blockIdx.x * 16 + ty;
            sb[tx][ty] = (tx < kleft && bc < p.N) ? B[(int64_t)bc * p.ldb + k0 + tx] : 0.f;
        } else {
            sb[ty][tx] = (ty < kleft && col < p.N) ? B[(int64_t)(k0 + ty) * p.ldb + col] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            sum += sa[ty][kk] * sb[kk][tx];
        __syncthreads();
    }
    if (row < p.M && col < p.N) {
        float *c = C + (int64_t)row * p.ldc + col;
        *c = finish(sum, p.alpha, p.beta, c, p.bias, col, p.act);
    }
}

// ---------------------------------------------------------------------------------
// Register micro-tile on the vector ALU: the technique of AutoMine++ #4 ("Let's use
// registers", "Matrix product by outer products of vectors") and Micro_gemm_4x4 ("FMA
// pattern", "Pipeline (double buffering)"), sized for 64-wide waves.
//
// A workgroup of 256 threads owns a 128 x 128 tile of C; thread (ty, tx) of the 16 x 16
// grid owns the 8 x 8 outputs at rows {ty*4 + i, 64 + ty*4 + i} and columns {tx*4 + j,
// 64 + tx*4 + j}, i, j < 4. Per K-tile of 8, op(A) and op(B) are staged in LDS k-major,
// As[k][m] and Bs[k][n], whatever their layout in memory, so that for each k a thread
// reads its 8 A and 8 B values as four 128-bit reads and adds their outer product to its
// 64 accumulators with 64 fused multiply-adds. Rows are padded to 132 floats, which keeps
// the transposing stores of plain A and transposed B free of bank conflicts. Global
// loads are one float per thread and element, consecutive threads on consecutive
// addresses, zero outside the matrix; the next K-tile's loads are in flight in
// registers while the current one is multiplied, with one barrier per K-tile. Any
// alignment; the epilogue is the same act(alpha*acc + beta*c + bias) as everywhere. (K-tiles
// of 16 would stage twice the elements, whose addresses the compiler keeps live across the
// loop; with two waves per SIMD that no longer fits the 256 registers and spills.)
// ---------------------------------------------------------------------------------
template <bool TA, bool TB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
sgemm_valu(GemmArgs p, int group_m)
{
    constexpr int BM = 128, BN = 128, BK = 8, LDS_ROW = 132, NT = 256;
    constexpr int PER_A = BM * BK / NT, PER_B = BK * BN / NT;    // elements staged per thread
    __shared__ __attribute__((aligned(16))) float As[2][BK][LDS_ROW];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDS_ROW];
    const int M = p.M, N = p.N, K = p.K;
    const float *__restrict__ A = p.A + (int64_t)blockIdx.z * p.strideA;
    const float *__restrict__ B = p.B + (int64_t)blockIdx.z * p.strideB;
    float *__restrict__ C = p.C + (int64_t)blockIdx.z * p.strideC;
    const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    int tm, tn;
    tile_coords(blockIdx.x, ceil_div(M, BM), ceil_div(N, BN), group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;

    // Element e = tid + NT * i of a tile, as (k, m) or (k, n): consecutive threads take
    // consecutive addresses of the operand as stored.
    auto a_coord = [&](int e, int &k, int &m) __attribute__((always_inline)) {
        if (TA) { m = e % BM; k = e / BM; } else { k = e % BK; m = e / BK; }
    };
    auto b_coord = [&](int e, int &k, int &n) __attribute__((always_inline)) {
        if (TB) { k = e % BK; n = e / BK; } else { n = e % BN; k = e / BN; }
    };
    // Loads are branch-free: an element outside the matrix reads the operand's first
    // element instead (always inside, since the product is not empty) and is replaced by
    // zero, so no load sits behind a branch that would keep registers live around it.
    float ra[PER_A], rb[PER_B];
    auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PER_A; ++i) {
            int k, m;
            a_coord(tid + NT * i, k, m);
            const int gm = m0 + m, gk = k0 + k;
            const bool in = gm < M && k < K - k0;          // no k0 + k overflow near K = 2^31
            const float v = A[in ? (TA ? (int64_t)gk * lda + gm : (int64_t)gm * lda + gk) : 0];
            ra[i] = in ? v : 0.f;
        }
#pragma unroll
        for (int i = 0; i < PER_B; ++i) {
            int k, n;
            b_coord(tid + NT * i, k, n);
            const int gn = n0 + n, gk = k0 + k;
            const bool in = k < K - k0 && gn < N;
            const float v = B[in ? (TB ? (int64_t)gn * ldb + gk : (int64_t)gk * ldb + gn) : 0];
            rb[i] = in ? v : 0.f;
        }
    };
    auto store = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PER_A; ++i) {
            int k, m;
            a_coord(tid + NT * i, k, m);
            As[st][k][m] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < PER_B; ++i) {
            int k, n;
            b_coord(tid + NT * i, k, n);
            Bs[st][k][n] = rb[i];
        }
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = 0.f;

    const int nk = ceil_div(K, BK);
    load(0);
    store(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int st = t & 1;
        if (t + 1 < nk)
            load((t + 1) * BK);          // in flight while this stage is multiplied
        // k's values are in registers while k+1's are read; the scheduling barrier after
        // each step keeps the compiler from hoisting every step's reads (and their 256
        // registers) to the top of the stage.
        floatx4 fa[2][2], fb[2][2];
        auto read = [&](int k, int buf) __attribute__((always_inline)) {
            fa[buf][0] = *reinterpret_cast<const floatx4 *>(&As[st][k][ty * 4]);
            fa[buf][1] = *reinterpret_cast<const floatx4 *>(&As[st][k][64 + ty * 4]);
            fb[buf][0] = *reinterpret_cast<const floatx4 *>(&Bs[st][k][tx * 4]);
            fb[buf][1] = *reinterpret_cast<const floatx4 *>(&Bs[st][k][64 + tx * 4]);
        };
        read(0, 0);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            if (k + 1 < BK)
                read(k + 1, (k + 1) & 1);
            const int buf = k & 1;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_fmaf(fa[buf][i / 4][i % 4], fb[buf][j / 4][j % 4], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t + 1 < nk)
            store(st ^ 1);               // the other stage: its last readers passed the previous barrier
        __syncthreads();
    }

    // Epilogue, one copy per activation (a uniform choice), so the 64 unrolled entries
    // carry no per-entry activation test.
    const float alpha = p.alpha, beta = p.beta;
    const bool has_bias = p.bias != nullptr;
    auto epilogue = [&](auto act_tag) __attribute__((always_inline)) {
        constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int gr = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + i - 4);
            if (gr >= M)
                continue;
            float *crow = C + (int64_t)gr * ldc;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int gc = n0 + (j < 4 ? tx * 4 + j : 64 + tx * 4 + j - 4);
                if (gc < N)
                    crow[gc] = finish_value(acc[i][j], alpha, beta, beta != 0.f ? crow[gc] : 0.f, has_bias,
                                            has_bias ? p.bias[gc] : 0.f, ACT);
            }
        }
    };
    if (p.act == ACT_GELU_TANH)
        epilogue(std::integral_constant<int, ACT_GELU_TANH>());
    else
        epilogue(std::integral_constant<int, ACT_NONE>());
}

// C = act(beta*C + bias) over the M x N window (C not read when beta == 0).
// Grid-stride in both dimensions; blockIdx.z selects the batch.
__global__ void __launch_bounds__(256) sgemm_scale(StridedArgs p)
{
    float *__restrict__ C = p.C + (int64_t)blockIdx.z * p.strideC;
    // 64-bit indices: the strides would carry a 32-bit index past 2^31 for M or N near it.
    for (int64_t i = blockIdx.y * blockDim.y + threadIdx.y; i < p.M; i += gridDim.y * blockDim.y)
        for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j < p.N; j += gridDim.x * blockDim.x) {
            float *c = C + i * p.ldc + j * p.incC;
            *c = finish(0.f, 0.f, p.beta, c, p.bias, (int)j, p.act);
        }
}

}  // namespace sgemm_impl
