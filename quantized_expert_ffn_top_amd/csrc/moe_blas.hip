// The plain bf16 GEMMs of the grouped-GEMM path (T > 16): router logits and
// the shared expert.  Dense bf16 x bf16 -> fp32 products with no routing, so
// they go to the rocBLAS library GEMM (Tensile kernels for gfx950); the bias
// and the SwiGLU run in small kernels of their own.
//
// rocBLAS is column-major: the row-major product C[M][N] = A[M][K] B[N][K]^T
// is the column-major C^T (N x M) = op_T(B as K x N) * A (as K x M).
//
// One handle per device, created on first use, atomics disallowed (the
// kernels it picks then sum in a fixed order: the same bits on every call).
// A mutex covers setting the handle's stream and enqueueing the product.

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {

namespace {

std::mutex g_blas_mu;
rocblas_handle g_blas[64];

// Row-major C[M][N] (fp32, ldc = N) = A[M][K] (bf16, lda = K) * B[N][K]^T (bf16, ldb = K).
// Returns the rocBLAS status (0: enqueued on st).
int gemm_bf16_f32(const uint16_t* A, const uint16_t* B, float* C, int M, int N, int K, hipStream_t st) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return rocblas_status_internal_error;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    if (!g_blas[dev]) {
        rocblas_handle h = nullptr;
        rocblas_status s = rocblas_create_handle(&h);
        if (s != rocblas_status_success) return s;
        s = rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
        if (s != rocblas_status_success) {
            rocblas_destroy_handle(h);
            return s;
        }
        g_blas[dev] = h;
    }
    rocblas_handle h = g_blas[dev];
    rocblas_status s = rocblas_set_stream(h, st);
    if (s != rocblas_status_success) return s;
    const float alpha = 1.f, beta = 0.f;
    return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &alpha,
                           B, rocblas_datatype_bf16_r, K, A, rocblas_datatype_bf16_r, K, &beta,
                           C, rocblas_datatype_f32_r, N, C, rocblas_datatype_f32_r, N,
                           rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
}

}  // namespace

// logits[t][e] += bias[e]
__global__ void k_add_bias(float* __restrict__ logits, const float* __restrict__ bias, int T, int E) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (int64_t)T * E) logits[i] += bias[i % E];
}

// a[t][o] = bf16_rne(silu(g) * u), u = ug[t][o], g = ug[t][Is + o]; silu(g) = g / (1 + e^-g)
__global__ void k_swiglu_bf16(const float* __restrict__ ug, int T, int Is, uint16_t* __restrict__ a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * Is) return;
    const int64_t t = i / Is, o = i - t * Is;
    const float u = ug[t * 2 * Is + o], g = ug[t * 2 * Is + Is + o];
    a[i] = (uint16_t)f32_to_bf16(g / (1.0f + expf(-g)) * u);
}

int launch_gemm_router(const uint16_t* x, int T, int H, int E, const uint16_t* w_r, const float* bias,
                       float* logits, hipStream_t st) {
    const int s = gemm_bf16_f32(x, w_r, logits, T, E, H, st);
    if (s != 0) return s;
    if (bias) {
        const int64_t n = (int64_t)T * E;
        k_add_bias<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(logits, bias, T, E);
    }
    return 0;
}

int launch_gemm_shared(const uint16_t* x, int T, int H, const uint16_t* sh_ug, const uint16_t* sh_down,
                       int Is, float* ug32, uint16_t* a_sh, float* y_sh, hipStream_t st) {
    int s = gemm_bf16_f32(x, sh_ug, ug32, T, 2 * Is, H, st);
    if (s != 0) return s;
    const int64_t n = (int64_t)T * Is;
    k_swiglu_bf16<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(ug32, T, Is, a_sh);
    return gemm_bf16_f32(a_sh, sh_down, y_sh, T, H, Is, st);
}

}  // namespace moe
