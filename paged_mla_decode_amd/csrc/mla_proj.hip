// The per-head projections on either side of the latent attention (SGLang v0.3
// MLA page, weight absorption; sglang-jax MLA gap page, sections 2.1-2.2):
//   q_abs[n, h, a] = sum_d q_nope[n, h, d] * W_UK[a, h, d]   (query side)
//   o[n, h, d]     = sum_a out[n, h, a]    * W_UV[a, h, d]   (output side)
//
// Both are, per head, D[n][m] = sum_k X[n][k] W[m][k] with the reduction index
// k contiguous in both operands as the kernel reads them (W_UK rows are a with
// d contiguous; W_UV rows are d with a contiguous). At decode batch sizes the
// weights and the 512-wide side are about equal in bytes and the arithmetic
// is small (an MFMA pass over them takes a fraction of the time HBM needs to
// deliver them), so the kernel is built to stream: every HBM access is a
// coalesced 16-byte lane load or store of whole row segments, and the bf16
// 32x32x16 MFMA reads its operands from LDS.
//
// Workgroup tile: 128 weight rows (m) by kNT activation rows (n), k in chunks
// of 128. Each chunk of both operands lands in LDS as rows of 256 bytes padded
// to 272, which keeps the 16-byte MFMA operand reads (eight rows per LDS pass)
// and the 16-byte staging writes free of bank conflicts. The next chunk is
// loaded into registers while the current one is multiplied. Wave w owns
// weight rows [32w, 32w + 32) and all kNT activation rows; its fp32 results
// go back through LDS as bf16 and leave as 256-byte row segments.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {
using namespace dev;

constexpr int kMT = 128;             // weight rows per workgroup
constexpr int kKC = 128;             // k per chunk
constexpr int kPitch = kKC * 2 + 16; // LDS bytes per staged row

template <int kNT, int kChunks>
__global__ __launch_bounds__(256) void head_gemm_kernel(const HeadGemmArgs g) {
    constexpr int kWBytes = kMT * kPitch;
    constexpr int kXBytes = kNT * kPitch;
    constexpr int kWLoads = kMT * (kKC / 8) / 256;  // 16-byte pieces per thread
    constexpr int kXLoads = kNT * (kKC / 8) / 256;
    constexpr int kNB = kNT / 32;
    static_assert(kNT * (kMT * 2 + 16) <= kWBytes + kXBytes, "output tile must fit the staging LDS");
    __shared__ __attribute__((aligned(16))) char lds[kWBytes + kXBytes];

    const int h = blockIdx.x, t = threadIdx.x;
    const int m_base = blockIdx.y * kMT, n_base = blockIdx.z * kNT;
    const int n_rows = g.n_rows;

    // Staging map: piece p of thread t is row t/16 + 16p, bytes 16*(t%16) of the chunk.
    const int srow = t >> 4, scol = t & 15;
    const uint16_t* wsrc = g.a + h * g.a_head + (int64_t)(m_base + srow) * g.a_row + 8 * scol;
    const int64_t w_step = 16 * g.a_row;
    const uint16_t* xsrc = g.b + h * g.b_head + 8 * scol;
    bf16x8 wreg[kWLoads], xreg[kXLoads];
    auto load = [&](int c) {
#pragma unroll
        for (int p = 0; p < kWLoads; ++p) wreg[p] = load_bf16x8(wsrc + p * w_step + kKC * c);
#pragma unroll
        for (int p = 0; p < kXLoads; ++p) {
            // Rows past the last one read the last row; their results are never stored.
            const int n = min(n_base + srow + 16 * p, n_rows - 1);
            xreg[p] = load_bf16x8(xsrc + (int64_t)n * g.b_row + kKC * c);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int p = 0; p < kWLoads; ++p)
            *reinterpret_cast<bf16x8*>(lds + (srow + 16 * p) * kPitch + 16 * scol) = wreg[p];
#pragma unroll
        for (int p = 0; p < kXLoads; ++p)
            *reinterpret_cast<bf16x8*>(lds + kWBytes + (srow + 16 * p) * kPitch + 16 * scol) = xreg[p];
    };

    const int lane = t & 63, w = t >> 6;
    const int r = lane & 31, gq = lane >> 5;
    const char* a_rd = lds + (32 * w + r) * kPitch + 16 * gq;
    const char* b_rd = lds + kWBytes + r * kPitch + 16 * gq;
    f32x16 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x16{};

    load(0);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c > 0) __syncthreads();  // every wave is done reading the previous chunk
        stage();
        if (c + 1 < kChunks) load(c + 1);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kKC / 16; ++s) {
            const bf16x8 A = *reinterpret_cast<const bf16x8*>(a_rd + 32 * s);
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const bf16x8 B = *reinterpret_cast<const bf16x8*>(b_rd + nb * 32 * kPitch + 32 * s);
                acc[nb] = mfma32(A, B, acc[nb]);
            }
        }
    }

    // D[m][n] of block nb sits at lane (n % 32, gq), register 4*r4 + i for
    // m = 32w + 8*r4 + 4*gq + i: four consecutive m, eight bytes of output row n.
    constexpr int kOutPitch = kMT * 2 + 16;
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const bf16x4 v = {(__bf16)acc[nb][4 * r4], (__bf16)acc[nb][4 * r4 + 1],
                              (__bf16)acc[nb][4 * r4 + 2], (__bf16)acc[nb][4 * r4 + 3]};
            *reinterpret_cast<bf16x4*>(lds + (32 * nb + r) * kOutPitch +
                                       2 * (32 * w + 8 * r4 + 4 * gq)) = v;
        }
    __syncthreads();
    __bf16* dst = reinterpret_cast<__bf16*>(g.d) + h * g.d_head + m_base + 8 * scol;
#pragma unroll
    for (int p = 0; p < kXLoads; ++p) {
        const int row = srow + 16 * p, n = n_base + row;
        if (n < n_rows)
            *reinterpret_cast<bf16x8*>(dst + (int64_t)n * g.d_row) =
                *reinterpret_cast<const bf16x8*>(lds + row * kOutPitch + 16 * scol);
    }
}

template <int kChunks>
void launch_nt(const HeadGemmArgs& g, int nt, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    if (nt == 32)
        head_gemm_kernel<32, kChunks><<<grid, block, 0, s>>>(g);
    else if (nt == 64)
        head_gemm_kernel<64, kChunks><<<grid, block, 0, s>>>(g);
    else
        head_gemm_kernel<128, kChunks><<<grid, block, 0, s>>>(g);
}

}  // namespace

int launch_head_gemm(const HeadGemmArgs& g, int num_heads, int m_len, int k_len, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (m_len % kMT != 0 || (k_len != 128 && k_len != 512)) return (int)hipErrorInvalidValue;
    // Activation tile: no taller than the rows need; at most 64 rows when k is a
    // single chunk (three workgroups per CU then hide the one load round trip;
    // with four chunks the register prefetch does, and 128 rows halve the
    // weight re-reads); and shrunk until the launch has a workgroup per CU of a
    // 256-CU device. Workgroups that share a weight tile sit heads*(m_len/128)
    // apart in launch order, a multiple of 8 when the head count is, so on one
    // XCD and its L2. (Measured at 128 heads, 32 to 1024 rows.)
    const int64_t tiles = (int64_t)num_heads * (m_len / kMT);
    int nt = k_len == 128 ? 64 : 128;
    while (nt > 32 && g.n_rows <= nt / 2) nt /= 2;
    while (nt > 32 && tiles * ((g.n_rows + nt - 1) / nt) < 256) nt /= 2;
    const dim3 grid(num_heads, m_len / kMT, (g.n_rows + nt - 1) / nt);
    if (k_len == 128)
        launch_nt<1>(g, nt, grid, s);
    else
        launch_nt<4>(g, nt, grid, s);
    return (int)hipGetLastError();
}

}  // namespace mla
