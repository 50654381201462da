// Device-side helpers shared by the decode kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace mla {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(8 * sizeof(unsigned)))) unsigned u32x8;
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kOverflowSlack = 64.0f;  // log2 units: probabilities stay below 2^64

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------

// Barriers written as inline assembly with a memory clobber, so that the
// compiler neither moves memory operations across them nor adds waits of its
// own. Direct-to-LDS loads complete in issue order with the other vector
// memory loads, so "vmcnt <= N" means everything but the N most recent loads
// has landed in LDS.
// The same wait for this wave alone, without the barrier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The wait that follows an item's page-index loads and its query loads: at
// most N vector memory operations outstanding. Loads retire in issue order, so
// when at least N loads were issued after the page-index loads, the indices
// have landed while the last N (query) loads may still be in flight. The
// trailing assembly comment tags it, so that a host test can check that
// invariant in the compiler's output (at least N vector loads between the
// last page-index load and this wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt_query() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0) ; mla-query-wait" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Wait until at most `pending` tiles of loads (kLoads instructions each) are
// outstanding, then a workgroup barrier. pending is wave-uniform, in [0, kMax].
template <int kMax, int kLoads>
__device__ __forceinline__ void wait_tiles_barrier(int pending) {
    if constexpr (kMax >= 1) {
        if (pending >= kMax) {
            wait_vmcnt_barrier<kMax * kLoads>();
            return;
        }
        wait_tiles_barrier<kMax - 1, kLoads>(pending);
    } else {
        wait_vmcnt_barrier<0>();
    }
}

// All of this wave's LDS accesses are complete, then a workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte direct global->LDS load: lane l's 16 bytes of src + kOff land at
// lds_base + kLdsAdd + 16 l. Issued as inline assembly so that the compiler's
// wait-count model never sees these LDS writes (it would otherwise drain every
// load before each LDS read); wait_vmcnt_barrier() orders them instead. M0
// holds the wave-uniform LDS address; one wait state separates its write from
// the load. kOff is the load's immediate offset and kLdsAdd a constant added to
// M0: one SALU write of M0 and no address arithmetic per load. The immediate offset moves the LDS
// destination too (lane l's 16 bytes land at M0 + offset + 16 l), so M0 gets
// kLdsAdd - kOff. A wave's blocks of one tile differ by such constants.
// kNT sets the non-temporal cache policy: for data read once per launch, so
// that it does not push out of the caches what is read again (queries shared
// by a row's pieces, partials the merge reads back).
// s_add_u32 also writes SCC (its carry): the statement declares it clobbered,
// or the compiler may keep a comparison's result in SCC across it and branch
// on the carry (tests/test_isa_scc.py checks the compiled kernels).
template <int kOff, int kLdsAdd, bool kNT = false>
__device__ __forceinline__ void dma16_imm(const void* src, uint32_t lds_base) {
    static_assert(kOff >= 0 && kOff < 4096, "13-bit signed immediate offset");
    if constexpr (kNT)
        asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3 nt"
                     :
                     : "s"(lds_base), "v"(src), "n"(kLdsAdd - kOff), "n"(kOff)
                     : "memory", "m0", "scc");
    else
        asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3"
                     :
                     : "s"(lds_base), "v"(src), "n"(kLdsAdd - kOff), "n"(kOff)
                     : "memory", "m0", "scc");
}

// dma16_imm with a wave-uniform base address in SGPRs and a 32-bit per-lane
// offset: lane l's 16 bytes of base + off + kOff land at M0 + kOff + 16 l, as
// above. For tiles whose tokens share one page, the page's address is uniform
// and the per-lane part is fixed, so no vector address arithmetic is needed.
template <int kOff, int kLdsAdd, bool kNT = false>
__device__ __forceinline__ void dma16_imm_s(const void* base, uint32_t off, uint32_t lds_base) {
    static_assert(kOff >= 0 && kOff < 4096, "13-bit signed immediate offset");
    if constexpr (kNT)
        asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%4 nt"
                     :
                     : "s"(lds_base), "v"(off), "s"(base), "n"(kLdsAdd - kOff), "n"(kOff)
                     : "memory", "m0", "scc");
    else
        asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%4"
                     :
                     : "s"(lds_base), "v"(off), "s"(base), "n"(kLdsAdd - kOff), "n"(kOff)
                     : "memory", "m0", "scc");
}

// 4-byte direct global->LDS load: lane l's dword lands at lds + 4 l. Same
// ordering rules as dma16_imm.
__device__ __forceinline__ void dma4(const void* src, LDS_AS void* dst) {
    const uint32_t lds = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "memory", "m0");
}

// Value held by lane ^ 32 / lane ^ 16, combined with the own value.
__device__ __forceinline__ float max_xor32(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Eight e4m3fn codes (two dwords) -> eight bf16 values, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned lo, unsigned hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// Software pipeline over N unrolled steps: the LDS operand of step i + D is
// requested right after step i's MFMA is issued, so D reads are in flight
// while the matrix core works. With one wave per SIMD there is no other wave
// to hide LDS latency behind, so this is what keeps the MFMA pipe busy.
template <int N, int D, int kReads, int kMfmas, class Load, class Use>
__device__ __forceinline__ void pipelined(Load load, Use use) {
    using Op = decltype(load(0));
    Op buf[D];
#pragma unroll
    for (int i = 0; i < D && i < N; ++i) buf[i] = load(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const Op cur = buf[i % D];
        use(i, cur);
        if (i + D < N) buf[i % D] = load(i + D);
    }
    // Pin the interleave: the prologue reads, then per step its MFMAs followed
    // by the reads D steps ahead (the scheduler would otherwise sink every read
    // next to its MFMA under register pressure).
    __builtin_amdgcn_sched_group_barrier(0x100, kReads * (D < N ? D : N), 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas, 0);
        if (i + D < N) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
    }
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x16 bf16 products issued as inline assembly. Volatile assembly keeps
// program order against other volatile assembly and against memory accesses,
// so a loop body can lay out its own interleave of independent MFMA chains and
// LDS reads. The compiler does not know these are matrix-core instructions and
// inserts none of their wait states, so:
//   * each starts with two wait states (an operand written by a VALU
//     instruction right before it is ready: the gfx950 VALU -> MFMA source
//     requirement), unless kWait is false: for operands that come from memory
//     (LDS or global loads), never from a VALU instruction. A host test
//     (tests/test_isa_hazards.py) checks the compiled kernels: no VALU
//     instruction writes a source of such an MFMA within four instructions
//     before it;
//   * back-to-back products accumulating into the same registers need none;
//   * readers (and VALU writers) of a result wait through a settle statement, at least
//     19 wait states after the last product that wrote it (an 8-pass XDL
//     write followed by a VALU access needs 11).
template <bool kWait = true>
__device__ __forceinline__ void mfma32_first_v(f32x16& c, bf16x8 a, bf16x8 b) {
    if constexpr (kWait)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
template <bool kWait = true>
__device__ __forceinline__ void mfma32_acc_v(f32x16& c, bf16x8 a, bf16x8 b) {
    if constexpr (kWait)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// c = 0 through the matrix core (0 . 0 + 0), so no VALU instruction writes c.
__device__ __forceinline__ void mfma32_zero_a(f32x16& c, bf16x8 z) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(c) : "v"(z));
}
template <bool kWait = true>
__device__ __forceinline__ void mfma32_acc_a(f32x16& c, bf16x8 a, bf16x8 b) {
    if constexpr (kWait)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// The fp8 score: 32x32x64 e4m3fn x e4m3fn (16 passes), 32 bytes of k per lane.
__device__ __forceinline__ void mfma32_f8_first_v(f32x16& c, u32x8 a, u32x8 b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_f8_acc_v(f32x16& c, u32x8 a, u32x8 b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// 24 wait states after the last MFMA that writes c, before any VALU access to
// it (a 16-pass XDL write needs 19, an 8-pass one 11).
__device__ __forceinline__ void settle_v(f32x16& c) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace dev
}  // namespace mla
