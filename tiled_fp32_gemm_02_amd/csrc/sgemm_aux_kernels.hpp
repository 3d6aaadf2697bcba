// The two small kernels of the library, included only by sgemm_api.hip:
//  - sgemm_tile16: the classic shared-memory kernel, one output per thread and 16x16
//    tiles (the GPT-2 post's hand-written matmul, "Tiled matrix multiplication"), kept
//    as the simplest correct rung and a baseline;
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
    for (int k0 = 0; k0 < p.K; k0 += 16) {
        if (TA) {   // thread (ty, tx) stages op(A)(block row + tx, k0 + ty): reads run along m
            const int ar = blockIdx.y * 16 + tx, ak = k0 + ty;
            sa[tx][ty] = (ar < p.M && ak < p.K) ? A[(int64_t)ak * p.lda + ar] : 0.f;
        } else {
            sa[ty][tx] = (row < p.M && k0 + tx < p.K) ? A[(int64_t)row * p.lda + k0 + tx] : 0.f;
        }
        if (TB) {   // thread (ty, tx) stages op(B)(k0 + tx, block col + ty): reads run along k
            const int bk = k0 + tx, bc = blockIdx.x * 16 + ty;
            sb[tx][ty] = (bk < p.K && bc < p.N) ? B[(int64_t)bc * p.ldb + bk] : 0.f;
        } else {
            sb[ty][tx] = (k0 + ty < p.K && col < p.N) ? B[(int64_t)(k0 + ty) * p.ldb + col] : 0.f;
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

// C = act(beta*C + bias) over the M x N window (C not read when beta == 0).
// Grid-stride in both dimensions; blockIdx.z selects the batch.
__global__ void __launch_bounds__(256) sgemm_scale(GemmArgs p)
{
    float *__restrict__ C = p.C + (int64_t)blockIdx.z * p.strideC;
    for (int i = blockIdx.y * blockDim.y + threadIdx.y; i < p.M; i += gridDim.y * blockDim.y)
        for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < p.N; j += gridDim.x * blockDim.x) {
            float *c = C + (int64_t)i * p.ldc + j;
            *c = finish(0.f, 0.f, p.beta, c, p.bias, j, p.act);
        }
}

}  // namespace sgemm_impl
