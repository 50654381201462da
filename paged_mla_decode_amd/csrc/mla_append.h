// Fused KV-cache append for the decode kernels: the work item that owns a
// request's last token first writes that token's cache row (latent, then
// rope) from the new-token inputs, in the cache's storage type. This is the
// fused cache update of the tpu-inference V2 MLA kernel (sglang-jax MLA gap
// page, section 2.4), with the nope and rope parts taken from separate inputs
// as the MLA token pool writes them (section 3.1).
#pragma once

#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace dev {

// fp32 -> OCP e4m3fn code (bias 7, three mantissa bits, largest finite 448),
// round to nearest, ties to even. |x| <= 448 and finite (the caller clamps).
__device__ __forceinline__ uint32_t e4m3fn_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t mag = b & 0x7FFFFFFFu;
    if (__uint_as_float(mag) < 0x1p-6f)  // subnormal codes: multiples of 2^-9 (8 -> 0x08, the smallest normal)
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
    // Rebias the exponent from 127 to 7 and round the 23-bit mantissa to 3 bits;
    // a carry out of the mantissa moves into the exponent, as it should.
    const uint32_t m = mag - ((127u - 7u) << 23);
    return sign | ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20);
}

__device__ __forceinline__ uint32_t e4m3fn_of(uint16_t bf16_bits, float kv_scale) {
    const float v = __uint_as_float((uint32_t)bf16_bits << 16);
    return e4m3fn_rne(fminf(fmaxf(__fdiv_rn(v, kv_scale), -448.f), 448.f));
}

// Writes row kv_end-1 of the item's request. Threads [0, nthreads) of the
// workgroup share the row: 72 pieces of 16 bytes (bf16) or 36 (fp8). The
// caller waits for the stores and synchronises the workgroup before the
// item's first tile load.
template <bool KV8>
__device__ __forceinline__ void append_row(const DecodeArgs& a, const mla_work_item& it, int tid,
                                           int nthreads) {
    constexpr int kRowBytes = KV8 ? 576 : 1152;
    const int tok = it.kv_end - 1;
    const int ps = a.page_size;
    const int pi = tok / ps;
    const int64_t slot = (int64_t)a.kv_indices[it.page_base + pi] * ps + (tok - pi * ps);
    uint8_t* dst = a.cache_w + slot * kRowBytes;
    const uint16_t* c = a.c_new + (int64_t)it.row * a.c_new_sn;
    const uint16_t* r = a.k_pe_new + (int64_t)it.row * a.k_pe_new_sn;
    if constexpr (!KV8) {
        for (int p = tid; p < 72; p += nthreads)
            *reinterpret_cast<bf16x8*>(dst + 16 * p) = load_bf16x8(p < 64 ? c + 8 * p : r + 8 * (p - 64));
    } else {
        for (int p = tid; p < 36; p += nthreads) {
            const uint16_t* src = p < 32 ? c + 16 * p : r + 16 * (p - 32);
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 8);
            u32x4 out;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u32x4 in = d < 2 ? lo : hi;
                const uint32_t w0 = in[(2 * d) % 4], w1 = in[(2 * d + 1) % 4];
                out[d] = e4m3fn_of(w0 & 0xFFFF, a.kv_scale) | e4m3fn_of(w0 >> 16, a.kv_scale) << 8 |
                         e4m3fn_of(w1 & 0xFFFF, a.kv_scale) << 16 | e4m3fn_of(w1 >> 16, a.kv_scale) << 24;
            }
            *reinterpret_cast<u32x4*>(dst + 16 * p) = out;
        }
    }
}

}  // namespace dev
}  // namespace mla
