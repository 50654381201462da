// The per-head projections on either side of the latent attention (SGLang v0.3
// MLA page, weight absorption; sglang-jax MLA gap page, sections 2.1-2.2):
//   q_abs[n, h, a] = sum_d q_nope[n, h, d] * W_UK[a, h, d]   (query side)
//   o[n, h, d]     = sum_a out[n, h, a]    * W_UV[a, h, d]   (output side)
//
// Both are, per head, a product whose reduction index is contiguous in both
// operands as the kernel reads them: the weight rows (W_UK in its [A, H, D]
// layout, W_UV per head transposed to [H, D, A]) are the A operand of the
// 32x32x16 bf16 MFMA and the activation rows its B operand, each lane loading
// 16 contiguous bytes straight from HBM (no LDS: every operand is used by one
// MFMA of one wave). D[m][n] = sum_k W[m][k] X[n][k] lands with four
// consecutive m per lane and register group, i.e. 8-byte runs of the output
// row n.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {
using namespace dev;

// Grid (heads, M / 128, ceil(N / 32)); wave w owns m in [128 y + 32 w, +32) and
// the workgroup's 32 rows n. K is kK (a compile-time multiple of 16).
template <int kK>
__global__ __launch_bounds__(256) void head_gemm_kernel(const HeadGemmArgs g) {
    constexpr int kSteps = kK / 16;
    constexpr int kRing = kSteps < 4 ? kSteps : 4;  // k-steps of operands in flight
    const int h = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 31, gq = lane >> 5;
    const int m0 = blockIdx.y * 128 + 32 * w;
    const int n0 = blockIdx.z * 32;
    // Rows past the last one read the last row (their results are not stored).
    const int n_ld = min(n0 + r, g.n_rows - 1);
    const uint16_t* arow = g.a + h * g.a_head + (int64_t)(m0 + r) * g.a_row + 8 * gq;
    const uint16_t* brow = g.b + h * g.b_head + (int64_t)n_ld * g.b_row + 8 * gq;

    bf16x8 A[kRing], B[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
        A[s] = load_bf16x8(arow + 16 * s);
        B[s] = load_bf16x8(brow + 16 * s);
    }
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        acc = mfma32(A[s % kRing], B[s % kRing], acc);
        if (s + kRing < kSteps) {
            A[s % kRing] = load_bf16x8(arow + 16 * (s + kRing));
            B[s % kRing] = load_bf16x8(brow + 16 * (s + kRing));
        }
    }
    const int n = n0 + r;
    if (n >= g.n_rows) return;
    __bf16* drow = reinterpret_cast<__bf16*>(g.d) + h * g.d_head + (int64_t)n * g.d_row + m0 + 4 * gq;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const bf16x4 v = {(__bf16)acc[4 * r4], (__bf16)acc[4 * r4 + 1], (__bf16)acc[4 * r4 + 2],
                          (__bf16)acc[4 * r4 + 3]};
        *reinterpret_cast<bf16x4*>(drow + 8 * r4) = v;
    }
}

}  // namespace

int launch_head_gemm(const HeadGemmArgs& g, int num_heads, int m_len, int k_len, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid(num_heads, m_len / 128, (g.n_rows + 31) / 32), block(256);
    if (k_len == 128)
        head_gemm_kernel<128><<<grid, block, 0, s>>>(g);
    else if (k_len == 512)
        head_gemm_kernel<512><<<grid, block, 0, s>>>(g);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace mla
