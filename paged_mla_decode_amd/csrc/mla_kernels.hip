// gfx950 (CDNA4, MI355X) kernels for weight-absorbed MLA decode over a paged
// latent cache, the log-sum-exp merge and the tree-suffix stable compaction.
//
// Decode kernel design (one workgroup per plan work item: a query row and a
// token chunk, all heads):
//   * Latent tiles of 32 tokens stream from HBM into LDS with 16-byte direct
//     global->LDS loads (no VGPR staging), double-buffered, with the page-table
//     lookups for tile i+2 and the loads of tile i+1 in flight while tile i is
//     computed. Unused rows of a partial last tile are redirected to a valid
//     row, so no load ever leaves the request's pages.
//   * The score is computed transposed, S^T[token, head] = C . Q^T, as an MFMA
//     with the absorbed query as the register-resident operand. The
//     accumulator then holds, per lane, one head and eight consecutive tokens:
//     exactly the operand layout the P . latent contraction needs, so the
//     probabilities never leave registers.
//   * The P . latent product reads the latent tile through the LDS transpose
//     load (ds_read_b64_tr_b16 / _b8), which hands each lane one latent column
//     over four (eight) consecutive tokens.
//   * Softmax in base 2 against a fixed reference point per head: the first
//     tile's max. The sum and O accumulate exp2(s - reference) and are never
//     rescaled, so O is only touched by MFMAs. Should a later score exceed the
//     reference by more than 2^64 (possible only for extreme score spreads),
//     the chunk is recomputed once with the true max as the reference. Either
//     way the result is the exact softmax, normalised at the end.
//   * Row max / sum across the lanes that share a head use v_permlane16/32_swap.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "mla_append.h"
#include "mla_device.h"
#include "mla_internal.h"
#include "mla_tile_layout.h"

namespace mla {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// The decode kernel
// ---------------------------------------------------------------------------

// Loads a wave issues after tile i's data when r = ntiles-1-i tiles follow it:
// the data of tiles i+1 .. i+stages-1 (kLoads each) and the page-table loads
// of the steps after the one that issued tile i's data, which fetch the
// entries of tiles i+stages+1 .. i+2 stages-1 (one each).
__host__ __device__ constexpr int wait_count(int r, int stages, int loads) {
    const int data = r < stages - 1 ? r : stages - 1;
    const int idx = r - stages < 0 ? 0 : (r - stages > stages - 1 ? stages - 1 : r - stages);
    return data * loads + idx;
}
// Waits until tile i's data (and every older load) has landed, then a
// workgroup barrier. r is wave-uniform and >= 0; wait_count is nondecreasing
// in r and constant from r = kR on.
template <int kR, int kStages, int kLoads>
__device__ __forceinline__ void wait_tile_and_idx(int r) {
    if constexpr (kR > 0) {
        if (r >= kR) {
            wait_vmcnt_barrier<wait_count(kR, kStages, kLoads)>();
            return;
        }
        wait_tile_and_idx<kR - 1, kStages, kLoads>(r);
    } else {
        wait_vmcnt_barrier<0>();
    }
}

template <int HW, int HS, bool KV8, bool OUT32, int MODE>
__global__ __launch_bounds__(64 * HS) void decode_kernel(const DecodeArgs a) {
    using L = TileLayout<KV8>;
    using SA = ScoreAddr<HW, KV8>;
    using PA = PvAddr<HW, KV8>;
    constexpr int NV = HW == 32 ? 16 : 8;                        // score values per lane per tile
    constexpr int kLoadsMax = (L::kNB + HS - 1) / HS;            // direct loads per wave per tile
    constexpr int kLoadsMin = L::kNB / HS;
    constexpr int kNTok = HS >= L::kNTB ? 1 : L::kNTB / HS;      // distinct tokens a lane loads
    constexpr int kSteps = SA::kSteps;
    constexpr int kDBlocks = PA::kDBlocks;
    static_assert(kNTok * L::kTPB <= 64, "one entry per lane");
    // LDS operand reads kept in flight ahead of the MFMAs.
    constexpr int kPipe = HW == 32 ? ((KV8 && OUT32) ? 2 : 4) : 3;
    // Ring of kStages tile buffers: tiles i+1 .. i+kStages-1 are in flight
    // while tile i is computed. Bounded by LDS and by the 6-bit vmcnt.
    constexpr int kStages = Stages<HW, HS, KV8, OUT32>::value;
    static_assert(wait_count(2 * kStages - 1, kStages, kLoadsMin) < 64, "vmcnt budget");
    // Page-table entries of tile t: issued kIdxLead steps before its data, in
    // slot t % kIdxSlots. A slot is rewritten two steps after its last read.
    constexpr int kIdxLead = kStages;
    constexpr int kIdxSlots = kIdxLead + 2;
    __shared__ __attribute__((aligned(1024))) char smem[kStages * L::kTileBytes];
    __shared__ __attribute__((aligned(16))) int idx_ring[kIdxSlots][HS][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Persistent worker: the plan's items [workers[w], workers[w+1]) in order.
    const int item_end = a.workers[blockIdx.x + 1];
    for (int item = a.workers[blockIdx.x]; item < item_end; ++item) {
        const mla_work_item it = a.items[item];
        const int ps = a.page_size;
        const int kv_begin = it.kv_begin;
        int kv_end = it.kv_end;
        if (a.kv_lens) kv_end = min(kv_end, a.kv_lens[it.request]);
        const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + kTile - 1) / kTile : 0;

        // Lane roles. hq: head (MFMA N index); gq: lane group along the K dim.
        const int hq = HW == 32 ? (lane & 31) : (lane & 15);
        const int gq = HW == 32 ? (lane >> 5) : (lane >> 4);
        // This lane's head, counted over the item's rows: rows it.row + r hold heads
        // r H .. r H + H - 1 (one row unless MLA_DECODE_SHARED_ROWS). Outputs,
        // partials and lse of consecutive rows are consecutive [H] blocks, so
        // it.row * H + head (it.partial * H + head) addresses them all.
        const int head = it.head_begin + w * HW + hq;
        // A wave whose heads lie past the item's only loads tiles: with 16 heads
        // the second wave halves the first one's loads per tile, which lets the
        // vmcnt budget cover twice the stages.
        const bool active = w * HW < it.num_rows * a.num_heads;

        // ---- absorbed query -> registers (B operand of the score MFMA) ----
        // Loaded with the first page-table entries (below), under one wait.
        bf16x8 q[kSteps];
        auto load_query = [&] {
            const int qrow = it.row + head / a.num_heads, qhead = head % a.num_heads;
            const uint16_t* qn = a.q_nope + (int64_t)qrow * a.qn_sn + (int64_t)qhead * a.qn_sh;
            const uint16_t* qr = a.q_rope + (int64_t)qrow * a.qr_sn + (int64_t)qhead * a.qr_sh;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const int k0 = (HW == 32 ? 16 : 32) * s + 8 * gq;
                q[s] = (s < kSteps * 8 / 9) ? load_bf16x8(qn + k0) : load_bf16x8(qr + (k0 - kLatent));
            }
        };
        if (MODE == kModeAppend && __builtin_amdgcn_readfirstlane(it.flags) & MLA_ITEM_LAST_CHUNK) {
            // Fused append: the request's new row goes to the cache before any
            // wave loads a tile that holds it.
            append_row<KV8>(a, it, threadIdx.x, 64 * HS);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the row's stores are done
            __syncthreads();
        }

        // ---- per-lane LDS bases (see mla_tile_layout.h) ----
        int sbase[SA::kBases], pbase[PA::kBases];
#pragma unroll
        for (int i = 0; i < SA::kBases; ++i) sbase[i] = SA::base(lane, i);
#pragma unroll
        for (int i = 0; i < PA::kBases; ++i) pbase[i] = PA::base(lane, i);
        // Global byte offset of the chunk this lane loads, within its row (chunk group 0).
        const int dma_lane_off = L::block_chunk(0, lane) * 16;

        // ---- page-table entries, through a small LDS ring ----
        // One direct-to-LDS dword load per wave and tile brings the entries of
        // the tokens the wave loads: lane kTPB k + j holds token j of its k-th
        // token block (tail tokens are clamped to the last valid token, so no
        // load leaves the request's pages). These loads are issued kIdxLead
        // steps ahead of the tile's data and are counted by the same vmcnt
        // waits. A scalar load of the entries would make the compiler wait
        // lgkmcnt(0), i.e. a full memory round trip, before the first LDS read
        // of every tile.
        const int32_t* page_table = a.kv_indices + it.page_base;
        auto page_of = [&](int tok) { return a.page_shift >= 0 ? tok >> a.page_shift : tok / ps; };
        auto issue_idx = [&](int tile) {
            const int k = min(lane / L::kTPB, kNTok - 1);
            const int tb = HS >= L::kNTB ? (w % L::kNTB) : (w + HS * k);
            const int j = min(lane - k * L::kTPB, L::kTPB - 1);
            const int tok = min(kv_begin + tile * kTile + tb * L::kTPB + j, kv_end - 1);
            dma4(page_table + page_of(tok), (LDS_AS int*)&idx_ring[tile % kIdxSlots][w][0]);
        };
        auto resolve_rows = [&](int tile, const uint8_t** rowp) {  // lane row pointers of a tile
            const int tstart = kv_begin + tile * kTile;
            const int slot = tile % kIdxSlots;
#pragma unroll
            for (int k = 0; k < kNTok; ++k) {
                const int tb = HS >= L::kNTB ? (w % L::kNTB) : (w + HS * k);
                const int tau = min(tstart + L::block_token(tb, lane), kv_end - 1);
                const int page = idx_ring[slot][w][k * L::kTPB + lane / L::kCG];
                const int row = a.page_shift >= 0 ? (tau & (ps - 1)) : tau % ps;
                rowp[k] = a.cache + ((int64_t)page * ps + row) * L::kRowBytes + dma_lane_off;
            }
        };
        // Load i of this wave is block b = w + HS i: token row k = i % kKs of the
        // wave, chunk group b / kNTB. With one row per wave (HS a multiple of
        // kNTB) that group is w / kNTB + (HS / kNTB) i; with kKs rows it is
        // i / kKs (w + HS k < kNTB). Either way a per-row base plus a
        // compile-time byte offset, and 1 KiB block b in LDS.
        auto issue_tile = [&](LDS_AS char* base, const uint8_t* const* rowp) {
            constexpr int kKs = HS >= L::kNTB ? 1 : L::kNTB / HS;
            static_assert(kKs == 1 ? HS % L::kNTB == 0 : HS * kKs == L::kNTB, "block geometry");
            const int wave_off = kKs == 1 ? (w / L::kNTB) * L::kCG * 16 : 0;
            const uint32_t lds0 = (uint32_t)(uintptr_t)(base + w * 1024);
            auto all = [&](auto nt_c) {
                [&]<int... I>(std::integer_sequence<int, I...>) {
                    ((L::kNB % HS == 0 || w + HS * I < L::kNB
                          ? dma16_imm<(kKs == 1 ? (HS / L::kNTB) * I : I / kKs) * L::kCG * 16, 1024 * HS * I,
                                      decltype(nt_c)::value>(rowp[I % kKs] + wave_off, lds0)
                          : (void)0),
                     ...);
                }(std::make_integer_sequence<int, kLoadsMax>{});
            };
            if (!KV8 && a.stream_tiles)
                all(std::true_type{});
            else
                all(std::false_type{});
        };

        // ---- accumulators ----
        f32x16 O32[HW == 32 ? kDBlocks : 1];
        f32x4 O16[HW == 16 ? kDBlocks : 1];
        // Softmax reference point (log2 units) per head: the first tile's max. The
        // running true max is tracked; if it ever exceeds the reference by more
        // than kOverflowSlack the chunk is recomputed with the true max as the
        // reference (which then bounds every probability by 1). O is only ever
        // touched by MFMAs inside the loop.
        float m_ref = -INFINITY, m_true = -INFINITY;
        float l_part = 0.f;
        __shared__ int rerun_flag[HS];

        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int i = 0; i < (HW == 32 ? kDBlocks : 1); ++i) O32[i] = f32x16{};
#pragma unroll
        for (int i = 0; i < (HW == 16 ? kDBlocks : 1); ++i) O16[i] = f32x4{};
        l_part = 0.f;

        if (ntiles > 0) {
            // The entries of tiles 0 .. kIdxLead-1, which steps read before the
            // loop's first wait; later ones come with the steps.
            for (int t = 0; t < kIdxLead && t < ntiles; ++t) issue_idx(t);
            // The query goes out beside them and one wait covers both (an item
            // without tiles needs no query). It must land before any tile load is
            // issued: the compiler does not see the tile loads, so its own waits
            // for these registers inside the loop would also drain the tiles in
            // flight.
            if (pass == 0 && active) load_query();
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            // One tile step. T is the buffer computed, N the one being filled;
            // distinct restrict-qualified parameters tell the compiler the two
            // never alias, so it adds no waits of its own for the direct-to-LDS
            // loads: the explicit vmcnt waits order them. Steps i < 0 only fill
            // the pipeline. Every vector memory load in flight here is a tile or
            // page-table load of this loop.
            auto tile_step = [&](const LDS_AS char* __restrict__ T, LDS_AS char* __restrict__ N, int i) {
                const int tstart = kv_begin + i * kTile;
                const int ahead = i + kStages - 1;  // the tile whose loads this step issues
                if (ahead < ntiles) {
                    const uint8_t* rowp[kNTok];
                    resolve_rows(ahead, rowp);
                    if (ahead + kIdxLead < ntiles) issue_idx(ahead + kIdxLead);
                    issue_tile(N, rowp);
                }
                if (i < 0) return;  // pipeline fill
                // Tile i has landed, and with it the entries that step i+1 reads.
                wait_tile_and_idx<2 * kStages - 1, kStages, kLoadsMin>(ntiles - 1 - i);

                const int nvalid = min(kTile, kv_end - tstart);
                if (active) {

                // ---- score: S^T = C . Q^T ----
                float sv[NV];
                if constexpr (HW == 32) {
                    f32x16 S = {};
                    auto load = [&](int s) -> bf16x8 {
                        const int off = sbase[SA::base_index(s, 0)] + SA::delta(s);
                        if constexpr (KV8) {
                            const i32x2 raw = *(const LDS_AS i32x2*)(T + off);
                            return fp8x8_to_bf16((unsigned)raw[0], (unsigned)raw[1]);
                        } else {
                            return *(const LDS_AS bf16x8*)(T + off);
                        }
                    };
                    pipelined<kSteps, kPipe, 1, 1>(load, [&](int s, bf16x8 A) { S = mfma32(A, q[s], S); });
#pragma unroll
                    for (int r = 0; r < 16; ++r) sv[r] = S[r];
                } else {
                    f32x4 S0 = {}, S1 = {};
                    struct Pair { bf16x8 a0, a1; };
                    auto load = [&](int s) -> Pair {
                        const int off0 = sbase[SA::base_index(s, 0)] + SA::delta(s);
                        const int off1 = sbase[SA::base_index(s, 1)] + SA::delta(s);
                        if constexpr (KV8) {
                            const i32x2 r0 = *(const LDS_AS i32x2*)(T + off0);
                            const i32x2 r1 = *(const LDS_AS i32x2*)(T + off1);
                            return {fp8x8_to_bf16((unsigned)r0[0], (unsigned)r0[1]),
                                    fp8x8_to_bf16((unsigned)r1[0], (unsigned)r1[1])};
                        } else {
                            return {*(const LDS_AS bf16x8*)(T + off0), *(const LDS_AS bf16x8*)(T + off1)};
                        }
                    };
                    pipelined<kSteps, kPipe, 2, 2>(load, [&](int s, Pair A) {
                        S0 = mfma16(A.a0, q[s], S0);
                        S1 = mfma16(A.a1, q[s], S1);
                    });
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        sv[r] = S0[r];
                        sv[4 + r] = S1[r];
                    }
                }

                // ---- scale, mask the tail, tile max ----
                float tmax = -INFINITY;
#pragma unroll
                for (int r = 0; r < NV; ++r) {
                    // token of value r: HW32: 16*(r/8) + 8*g + r%8; HW16: 8*g + r
                    const int tok = HW == 32 ? (16 * (r >> 3) + 8 * gq + (r & 7)) : (8 * gq + r);
                    float v = sv[r] * a.scale_log2;
                    v = tok < nvalid ? v : -INFINITY;
                    sv[r] = v;
                    tmax = fmaxf(tmax, v);
                }
                if (HW == 16) tmax = max_xor16(tmax);
                tmax = max_xor32(tmax);
                if (pass == 0 && i == 0) m_ref = tmax;
                m_true = fmaxf(m_true, tmax);

                // ---- probabilities relative to the reference ----
                float p[NV];
#pragma unroll
                for (int r = 0; r < NV; ++r) {
                    p[r] = fast_exp2(sv[r] - m_ref);
                    l_part += p[r];
                }

                // ---- O^T += C^T . P^T ----
                constexpr int kKK = HW == 32 ? 2 : 1;
                bf16x8 P[kKK], Plo[kKK];
#pragma unroll
                for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        P[kk][e] = (__bf16)p[8 * kk + e];
                        if (OUT32) Plo[kk][e] = (__bf16)(p[8 * kk + e] - (float)P[kk][e]);
                    }
                // Step j covers output block md = j % kDBlocks of token half kk = j / kDBlocks.
                auto load_pv = [&](int j) -> bf16x8 {
                    const int md = j % kDBlocks, kk = j / kDBlocks;
                    const int pb = pbase[PA::base_index(md)];
                    if constexpr (KV8) {
                        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (LDS_AS i32x2*)(T + pb + PA::delta(md, kk, 0)));
                        return fp8x8_to_bf16((unsigned)raw[0], (unsigned)raw[1]);
                    } else {
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (LDS_AS i16x4*)(T + pb + PA::delta(md, kk, 0)));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (LDS_AS i16x4*)(T + pb + PA::delta(md, kk, 1)));
                        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                };
                pipelined<kKK * kDBlocks, kPipe, KV8 ? 1 : 2, OUT32 ? 2 : 1>(load_pv, [&](int j, bf16x8 A) {
                    const int md = j % kDBlocks, kk = j / kDBlocks;
                    if constexpr (HW == 32) {
                        O32[md] = mfma32(A, P[kk], O32[md]);
                        if (OUT32) O32[md] = mfma32(A, Plo[kk], O32[md]);
                    } else {
                        O16[md] = mfma16(A, P[kk], O16[md]);
                        if (OUT32) O16[md] = mfma16(A, Plo[kk], O16[md]);
                    }
                });
                }  // active
                lds_barrier();  // everyone is done with this buffer before it is refilled
            };
            // Tile t lives in buffer t % kStages. Step i computes tile i and fills
            // the buffer of tile i-1 (freed by the previous step) with tile
            // i + kStages - 1; steps i < 0 only fill the pipeline.
            int cur = 1 % kStages;  // buffer of tile -(kStages-1)
            for (int i = -(kStages - 1); i < ntiles; ++i) {
                const int nxt = cur == 0 ? kStages - 1 : cur - 1;  // buffer of tile i-1 = tile i+kStages-1
                tile_step((const LDS_AS char*)smem + cur * L::kTileBytes,
                          (LDS_AS char*)smem + nxt * L::kTileBytes, i);
                cur = cur + 1 == kStages ? 0 : cur + 1;
            }
        }
        // Did any head of the workgroup outgrow its reference? All waves must agree,
        // since the tiles are loaded cooperatively.
        const bool over = __builtin_amdgcn_ballot_w64(m_true > m_ref + kOverflowSlack) != 0;
        if (lane == 0) rerun_flag[w] = over ? 1 : 0;
        lds_barrier();
        int any = 0;
#pragma unroll
        for (int k = 0; k < HS; ++k) any |= rerun_flag[k];
        lds_barrier();
        if (!any) break;
        m_ref = m_true;  // second pass: every probability is at most 1
        }

        if (!active) continue;  // a load-only wave has no heads to write

        // ---- finalize: l across the lanes of a head, normalise, write ----
        const float m_run = m_ref;
        float l = l_part;
        if (HW == 16) l = sum_xor16(l);
        l = sum_xor32(l);
        const bool empty = !(l > 0.f);
        float inv = empty ? 0.f : (a.out_scale / l);
        float lse = empty ? -INFINITY : (m_run + __log2f(l)) * kLn2;
        const int nh = a.num_heads;
        // Fused prefix merge of an unsplit row: out = wa * prefix + wb * this,
        // with the weights of the two states' LSE merge; lse becomes theirs.
        const bool fuse = MODE == kModeMerge && it.partial < 0;
        float wa = 0.f;
        if (MODE == kModeMerge && fuse) {
            const float la = a.prefix_lse[(int64_t)it.row * nh + head];
            float wb = 0.f, s = -INFINITY;
            if (!(la == -INFINITY && lse == -INFINITY)) {
                const float mx = fmaxf(la, lse);
                const float ea = __expf(la - mx), eb = __expf(lse - mx);
                wa = ea / (ea + eb);
                wb = eb / (ea + eb);
                s = mx + __logf(ea + eb);
            }
            inv *= wb;
            lse = s;
        }
        // Adds the prefix's share to four consecutive output columns.
        auto with_prefix = [&](f32x4 x, int64_t off) -> f32x4 {
            if (MODE == kModeMerge && fuse) {
                if constexpr (OUT32) {
                    x += wa * *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.prefix_out) + off);
                } else {
                    const bf16x4 p = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(a.prefix_out) + off);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] += wa * (float)p[e];
                }
            }
            return x;
        };

        if (it.partial >= 0 && OUT32) {
            float* po = reinterpret_cast<float*>(a.part_out) + ((int64_t)it.partial * nh + head) * kLatent;
            if constexpr (HW == 32) {
#pragma unroll
                for (int md = 0; md < kDBlocks; ++md)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int d = 32 * md + 8 * r4 + 4 * gq;
                        f32x4 v = {O32[md][4 * r4] * inv, O32[md][4 * r4 + 1] * inv,
                                   O32[md][4 * r4 + 2] * inv, O32[md][4 * r4 + 3] * inv};
                        *reinterpret_cast<f32x4*>(po + d) = v;
                    }
            } else {
#pragma unroll
                for (int md = 0; md < kDBlocks; ++md) {
                    const int d = 16 * md + 4 * gq;
                    *reinterpret_cast<f32x4*>(po + d) = O16[md] * inv;
                }
            }
            if (gq == 0) a.part_lse[(int64_t)it.partial * nh + head] = lse;
        } else {
            // bf16 partials (bf16 output) take the same path as the output itself.
            const int64_t orow = it.partial >= 0 ? (int64_t)it.partial * nh + head : (int64_t)it.row * nh + head;
            void* obase = it.partial >= 0 ? a.part_out : a.out;
            if constexpr (OUT32) {
                float* o = reinterpret_cast<float*>(obase) + orow * kLatent;
                if constexpr (HW == 32) {
#pragma unroll
                    for (int md = 0; md < kDBlocks; ++md)
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int d = 32 * md + 8 * r4 + 4 * gq;
                            f32x4 v = {O32[md][4 * r4] * inv, O32[md][4 * r4 + 1] * inv,
                                       O32[md][4 * r4 + 2] * inv, O32[md][4 * r4 + 3] * inv};
                            *reinterpret_cast<f32x4*>(o + d) = with_prefix(v, orow * kLatent + d);
                        }
                } else {
#pragma unroll
                    for (int md = 0; md < kDBlocks; ++md) {
                        const int d = 16 * md + 4 * gq;
                        *reinterpret_cast<f32x4*>(o + d) = with_prefix(O16[md] * inv, orow * kLatent + d);
                    }
                }
            } else {
                __bf16* o = reinterpret_cast<__bf16*>(obase) + orow * kLatent;
                if constexpr (HW == 32) {
#pragma unroll
                    for (int md = 0; md < kDBlocks; ++md)
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int d = 32 * md + 8 * r4 + 4 * gq;
                            f32x4 x = {O32[md][4 * r4] * inv, O32[md][4 * r4 + 1] * inv,
                                       O32[md][4 * r4 + 2] * inv, O32[md][4 * r4 + 3] * inv};
                            x = with_prefix(x, orow * kLatent + d);
                            bf16x4 v = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
                            *reinterpret_cast<bf16x4*>(o + d) = v;
                        }
                } else {
#pragma unroll
                    for (int md = 0; md < kDBlocks; ++md) {
                        const int d = 16 * md + 4 * gq;
                        const f32x4 x = with_prefix(O16[md] * inv, orow * kLatent + d);
                        bf16x4 v = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
                        *reinterpret_cast<bf16x4*>(o + d) = v;
                    }
                }
            }
            if (gq == 0) {
                if (it.partial >= 0)
                    a.part_lse[orow] = lse;
                else if (a.lse)
                    a.lse[orow] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of split-KV partials (one wave per (row, head)).
// ---------------------------------------------------------------------------
// Running LSE combination of one head's partials: m (max lse so far), wsum
// (sum of e^{lse - m}) and acc (sum of e^{lse - m} v, 8 columns per lane).
struct MergeState {
    float m = -INFINITY, wsum = 0.f;
    f32x8 acc = {};
};

// Folds partials [p0, p0 + nb) (nb <= kBatch) of merge `mi`, head h, into st.
// The batch's loads are all in flight before any is combined; a larger
// maximum rescales what came before.
template <bool OUT32, int kBatch>
__device__ __forceinline__ void merge_batch(const MergePartialsArgs& a, const mla_merge_item& mi, int h,
                                            int lane, int p0, int nb, MergeState& st) {
    using V = std::conditional_t<OUT32, f32x8, bf16x8>;
    const int nh = a.num_heads;
    float l[kBatch];
    V v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        if (k < nb) {
            const int64_t slot = (int64_t)(mi.partial_begin + (p0 + k) * mi.partial_stride) * nh + h;
            l[k] = a.part_lse[slot];
            v[k] = *(reinterpret_cast<const V*>(a.part_out) + slot * (kLatent / 8) + lane);
        }
    }
    float mb = st.m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
        if (k < nb) mb = fmaxf(mb, l[k]);
    if (mb == -INFINITY) return;  // every partial so far is empty
    const float r = st.m == -INFINITY ? 0.f : fast_exp2((st.m - mb) * kLog2e);
    st.acc = st.acc * r;
    st.wsum *= r;
    st.m = mb;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        if (k < nb) {
            const float wp = fast_exp2((l[k] - st.m) * kLog2e);
            st.wsum += wp;
            f32x8 x;
            if constexpr (OUT32) {
                x = v[k];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (float)v[k][e];
            }
            st.acc += wp * x;
        }
    }
}

// Folds the given prefix state of (row, h) into st: the fused prefix merge of
// a split row. Lane reads its 8 columns before merge_store writes them, so the
// output may be the prefix's own memory.
template <bool OUT32>
__device__ __forceinline__ void merge_prefix(const MergePartialsArgs& a, int row, int h, int lane,
                                             MergeState& st) {
    using V = std::conditional_t<OUT32, f32x8, bf16x8>;
    const int64_t i = (int64_t)row * a.num_heads + h;
    const float l = a.prefix_lse[i];
    if (l == -INFINITY) return;
    const V v = *(reinterpret_cast<const V*>(a.prefix_out) + i * (kLatent / 8) + lane);
    const float mb = fmaxf(st.m, l);
    const float r = st.m == -INFINITY ? 0.f : fast_exp2((st.m - mb) * kLog2e);
    st.acc = st.acc * r;
    st.wsum *= r;
    st.m = mb;
    const float wp = fast_exp2((l - mb) * kLog2e);
    st.wsum += wp;
    f32x8 x;
    if constexpr (OUT32) {
        x = v;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
    }
    st.acc += wp * x;
}

template <bool OUT32>
__device__ __forceinline__ void merge_store(const MergePartialsArgs& a, const mla_merge_item& mi, int h, int lane,
                                            const MergeState& st) {
    const int nh = a.num_heads;
    const bool empty = !(st.wsum > 0.f);
    const float inv = empty ? 0.f : 1.f / st.wsum;
    const int64_t orow = (int64_t)mi.row * nh + h;
    if constexpr (OUT32) {
        *reinterpret_cast<f32x8*>(reinterpret_cast<float*>(a.out) + orow * kLatent + 8 * lane) = st.acc * inv;
    } else {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (__bf16)(st.acc[e] * inv);
        *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(a.out) + orow * kLatent + 8 * lane) = o;
    }
    if (a.lse && lane == 0) a.lse[orow] = empty ? -INFINITY : st.m + __logf(st.wsum);
}

// Few partials per row: one wave per (row, head) folds them all. For plans
// without wide merges (graph-safe launches and plans with wide merges take
// merge_partials_mixed_kernel).
template <bool OUT32>
__global__ __launch_bounds__(256) void merge_partials_kernel(const MergePartialsArgs a) {
    constexpr int kBatch = 8;
    const mla_merge_item mi = a.merges[blockIdx.x];
    const int lane = threadIdx.x & 63;
    for (int h = blockIdx.y * 4 + (threadIdx.x >> 6); h < a.num_heads; h += gridDim.y * 4) {
        MergeState st;
        for (int p0 = 0; p0 < mi.num_partials; p0 += kBatch)
            merge_batch<OUT32, kBatch>(a, mi, h, lane, p0, min(kBatch, mi.num_partials - p0), st);
        if (a.prefix_lse) merge_prefix<OUT32>(a, mi.row, h, lane, st);
        merge_store<OUT32>(a, mi, h, lane, st);
    }
}

// Many partials per row (a very long request cut into hundreds of pieces): a
// workgroup of kWaves waves per (row, head), each folding its own batches, the
// wave states combined through LDS. One wave alone would wait out hundreds of
// dependent memory round trips. The same launch merges the narrow rows that
// follow the wide ones in the plan (kWaves heads per workgroup, one wave per
// head, as merge_partials_kernel does), so that a plan with both kinds costs
// one merge launch: workgroups [0, wide_bound * H) take (wide merge, head),
// the rest (narrow merge, 16 heads).
template <bool OUT32>
__global__ __launch_bounds__(1024) void merge_partials_mixed_kernel(const MergePartialsArgs a) {
    constexpr int kWaves = 16, kBatch = 8;
    const int nh = a.num_heads;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int num_wide = a.dev_num_wide ? *a.dev_num_wide : a.num_wide;
    const int num_merges = a.dev_num_merges ? *a.dev_num_merges : a.num_merges;
    const int wide_blocks = a.wide_bound * nh;
    if ((int)blockIdx.x >= wide_blocks) {
        const int b = blockIdx.x - wide_blocks, per = (nh + kWaves - 1) / kWaves;
        const int m = num_wide + b / per, h = (b % per) * kWaves + wv;
        if (m >= num_merges || h >= nh) return;
        const mla_merge_item mi = a.merges[m];
        MergeState st;
        for (int p0 = 0; p0 < mi.num_partials; p0 += kBatch)
            merge_batch<OUT32, kBatch>(a, mi, h, lane, p0, min(kBatch, mi.num_partials - p0), st);
        if (a.prefix_lse) merge_prefix<OUT32>(a, mi.row, h, lane, st);
        merge_store<OUT32>(a, mi, h, lane, st);
        return;
    }
    const int m = blockIdx.x / nh, h = blockIdx.x % nh;
    if (m >= num_wide) return;  // graph-safe launch: past this plan's wide merges
    const mla_merge_item mi = a.merges[m];
    MergeState st;
    for (int p0 = wv * kBatch; p0 < mi.num_partials; p0 += kWaves * kBatch)
        merge_batch<OUT32, kBatch>(a, mi, h, lane, p0, min(kBatch, mi.num_partials - p0), st);
    __shared__ float sm[kWaves], sw[kWaves];
    __shared__ f32x8 sacc[kWaves][64];
    if (lane == 0) {
        sm[wv] = st.m;
        sw[wv] = st.wsum;
    }
    sacc[wv][lane] = st.acc;
    __syncthreads();
    if (wv != 0) return;
    MergeState t;
    for (int k = 0; k < kWaves; ++k) t.m = fmaxf(t.m, sm[k]);
    if (t.m != -INFINITY) {
        for (int k = 0; k < kWaves; ++k) {
            if (sm[k] == -INFINITY) continue;
            const float r = fast_exp2((sm[k] - t.m) * kLog2e);
            t.wsum += r * sw[k];
            t.acc += r * sacc[k][lane];
        }
    }
    if (a.prefix_lse) merge_prefix<OUT32>(a, mi.row, h, lane, t);
    merge_store<OUT32>(a, mi, h, lane, t);
}

// ---------------------------------------------------------------------------
// Two-state LSE merge (one wave per row, 8 elements per lane per step).
// ---------------------------------------------------------------------------
template <bool F32>
__global__ __launch_bounds__(256) void merge_states_kernel(const void* va, const float* sa,
                                                           const void* vb, const float* sb,
                                                           void* vo, float* so, int64_t rows,
                                                           int d) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float a = sa[row], b = sb[row];
    float wa = 0.f, wb = 0.f, s = -INFINITY;
    if (!(a == -INFINITY && b == -INFINITY)) {
        const float m = fmaxf(a, b);
        const float ea = __expf(a - m), eb = __expf(b - m);
        const float sum = ea + eb;
        wa = ea / sum;
        wb = eb / sum;
        s = m + __logf(sum);
    }
    for (int c = 8 * lane; c < d; c += 512) {
        const int64_t off = row * d + c;
        if constexpr (F32) {
            const f32x8 x = *reinterpret_cast<const f32x8*>(reinterpret_cast<const float*>(va) + off);
            const f32x8 y = *reinterpret_cast<const f32x8*>(reinterpret_cast<const float*>(vb) + off);
            *reinterpret_cast<f32x8*>(reinterpret_cast<float*>(vo) + off) = wa * x + wb * y;
        } else {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(va) + off);
            const bf16x8 y = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(vb) + off);
            bf16x8 r;
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = (__bf16)(wa * (float)x[e] + wb * (float)y[e]);
            *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(vo) + off) = r;
        }
    }
    if (lane == 0) so[row] = s;
}

// ---------------------------------------------------------------------------
// Tree-suffix stable compaction (one wave per query row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tree_compact_kernel(
    const uint8_t* __restrict__ mask, int64_t mask_stride, const int32_t* __restrict__ req_to_token,
    int64_t req_stride, const int32_t* __restrict__ prefix_lens, int width, int num_rows,
    int num_actual_rows, int32_t* __restrict__ table, int64_t table_stride,
    int32_t* __restrict__ seqlens) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= num_rows) return;
    const int lane = threadIdx.x & 63;
    int32_t* trow = table + (int64_t)row * table_stride;
    if (row >= num_actual_rows) {  // graph padding: read no mask
        for (int c = lane; c < width; c += 64) trow[c] = 0;
        if (lane == 0) seqlens[row] = 0;
        return;
    }
    const int req = row / width;
    const int32_t* slots = req_to_token + (int64_t)req * req_stride + prefix_lens[req];
    const uint8_t* mrow = mask + (int64_t)row * mask_stride;
    int count = 0;
    for (int seg = 0; seg < width; seg += 64) {
        const int c = seg + lane;
        const bool v = c < width && mrow[c] != 0;
        count += __popcll(__builtin_amdgcn_ballot_w64(v));
    }
    const uint64_t le = (uint64_t(2) << lane) - 1;  // lanes 0..lane
    int before = 0;
    for (int seg = 0; seg < width; seg += 64) {
        const int c = seg + lane;
        const bool v = c < width && mrow[c] != 0;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(v);
        const int rank = before + __popcll(bal & le);  // inclusive count of visible columns
        if (c < width) {
            const int dest = v ? rank - 1 : count + c - rank;
            trow[dest] = slots[c];
        }
        before += __popcll(bal);
    }
    if (lane == 0) seqlens[row] = count;
}

// ---------------------------------------------------------------------------
// Query quantisation for the fp8 score. One wave per (row, head): workgroup
// (row, g) takes heads 4 g .. 4 g + 3. Per head, lane l holds the eight values of 16-byte
// chunk l of the 576 (no-rope chunks 0..63) and, for l < 8, rope chunk l as
// well. amax over the head's values fixes e, the smallest integer with
// amax * 2^-e <= 448 (0 for a head of zeros); each value is scaled by 2^-e
// (exact) and rounded to its nearest e4m3fn code.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_at(const bf16x8& v, int i) { return (float)v[i]; }

__global__ __launch_bounds__(256) void quantize_query_kernel(const QuantQueryArgs q) {
    const int row = blockIdx.x;
    if (row >= *q.dev_num_rows) return;
    const int lane = threadIdx.x & 63;
    const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
    if (h < q.num_heads) {
        const bf16x8 vn = load_bf16x8(q.q_nope + (int64_t)row * q.qn_sn + (int64_t)h * q.qn_sh + 8 * lane);
        bf16x8 vr = {};
        if (lane < kRope / 8) vr = load_bf16x8(q.q_rope + (int64_t)row * q.qr_sn + (int64_t)h * q.qr_sh + 8 * lane);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_at(vn, i)), fabsf(bf16_at(vr, i))));
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
        // amax = m * 2^k with m in [0.5, 1); 448 = 0.875 * 2^9.
        int k = 0;
        const float m = frexpf(amax, &k);
        const int e = amax > 0.f ? (m <= 0.875f ? k - 9 : k - 8) : 0;
        auto pack = [&](const bf16x8& v) {
            uint2 r;
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = e4m3fn_rne(ldexpf(bf16_at(v, i), -e));
            r.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            r.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
            return r;
        };
        uint8_t* dst = q.codes + ((int64_t)row * q.num_heads + h) * kRow;
        *reinterpret_cast<uint2*>(dst + 8 * lane) = pack(vn);
        if (lane < kRope / 8) *reinterpret_cast<uint2*>(dst + kLatent + 8 * lane) = pack(vr);
        if (lane == 0) q.exps[(int64_t)row * q.num_heads + h] = e;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int launch_quantize_query(const QuantQueryArgs& q, int rows, void* stream) {
    quantize_query_kernel<<<dim3(rows, (q.num_heads + 3) / 4), dim3(256), 0, (hipStream_t)stream>>>(q);
    return (int)hipGetLastError();
}

template <int HW, int HS>
static int launch_decode_hs(int kv_dtype, int out_dtype, const DecodeArgs& a, int n, hipStream_t s) {
    const dim3 grid(n), block(64 * HS);
    const bool kv8 = kv_dtype == MLA_DTYPE_FP8_E4M3FN;
    const bool o32 = out_dtype == MLA_DTYPE_FP32;
    // The fused append and prefix merge are instantiations of their own. The
    // single-pass tree verify exists for the 128-head kernel only.
    if (a.sfx_table) return (int)hipErrorInvalidValue;
    const int mode = a.c_new ? kModeAppend : a.prefix_lse ? kModeMerge : kModePlain;
    auto go = [&](auto kv8_t, auto o32_t) {
        constexpr bool K = decltype(kv8_t)::value, O = decltype(o32_t)::value;
        if (mode == kModeAppend)
            decode_kernel<HW, HS, K, O, kModeAppend><<<grid, block, 0, s>>>(a);
        else if (mode == kModeMerge)
            decode_kernel<HW, HS, K, O, kModeMerge><<<grid, block, 0, s>>>(a);
        else
            decode_kernel<HW, HS, K, O, kModePlain><<<grid, block, 0, s>>>(a);
    };
    using T = std::true_type;
    using F = std::false_type;
    if (kv8 && o32)
        go(T{}, T{});
    else if (kv8)
        go(T{}, F{});
    else if (o32)
        go(F{}, T{});
    else
        go(F{}, F{});
    return (int)hipGetLastError();
}

int launch_decode(const Variant& v, int kv_dtype, int out_dtype, const DecodeArgs& a, int num_workers,
                  void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (num_workers <= 0) return 0;
    if (v.hw == 32 && v.hs == 4) return launch_decode_h128(kv_dtype, out_dtype, a, num_workers, stream);
    if (v.hw == 16 && v.hs == 1) return launch_decode_hs<16, 1>(kv_dtype, out_dtype, a, num_workers, s);
    if (v.hw == 16 && v.hs == 2) return launch_decode_hs<16, 2>(kv_dtype, out_dtype, a, num_workers, s);
    if (v.hw == 16 && v.hs == 4) return launch_decode_hs<16, 4>(kv_dtype, out_dtype, a, num_workers, s);
    return (int)hipErrorInvalidValue;
}

int launch_merge_partials(int out_dtype, const MergePartialsArgs& a, int num_merges, int num_wide,
                          void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const bool o32 = out_dtype == MLA_DTYPE_FP32;
    const int nh = a.num_heads;
    if (!a.dev_num_merges && num_merges <= 0) return 0;
    if (a.dev_num_merges || num_wide > 0) {
        // One launch for the wide merges and the narrow ones after them.
        // Graph-safe: num_merges and num_wide bound the plan's counts, which the
        // kernel reads from its device copy; any of the merges may be narrow.
        MergePartialsArgs m = a;
        m.wide_bound = num_wide;
        m.num_wide = num_wide;
        m.num_merges = num_merges;
        const int narrow = a.dev_num_merges ? num_merges : num_merges - num_wide;
        const int blocks = num_wide * nh + narrow * ((nh + 15) / 16);
        if (blocks <= 0) return 0;
        if (o32)
            merge_partials_mixed_kernel<true><<<blocks, 1024, 0, s>>>(m);
        else
            merge_partials_mixed_kernel<false><<<blocks, 1024, 0, s>>>(m);
        return (int)hipGetLastError();
    }
    const dim3 grid(num_merges, (nh + 3) / 4), block(256);
    if (o32)
        merge_partials_kernel<true><<<grid, block, 0, s>>>(a);
    else
        merge_partials_kernel<false><<<grid, block, 0, s>>>(a);
    return (int)hipGetLastError();
}

int launch_merge_states(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                        void* v_out, float* s_out, int64_t num_rows, int32_t head_dim,
                        int32_t v_dtype, void* stream) {
    if (num_rows <= 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)((num_rows + 3) / 4)), block(256);
    if (v_dtype == MLA_DTYPE_FP32)
        merge_states_kernel<true><<<grid, block, 0, s>>>(v_a, s_a, v_b, s_b, v_out, s_out, num_rows, head_dim);
    else
        merge_states_kernel<false><<<grid, block, 0, s>>>(v_a, s_a, v_b, s_b, v_out, s_out, num_rows, head_dim);
    return (int)hipGetLastError();
}

int launch_tree_compact(const uint8_t* mask, int64_t mask_stride, const int32_t* req_to_token,
                        int64_t req_stride, const int32_t* prefix_lens, int32_t width,
                        int32_t num_rows, int32_t num_actual_rows, int32_t* page_table,
                        int64_t table_stride, int32_t* seqlens, void* stream) {
    if (num_rows <= 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((num_rows + 3) / 4), block(256);
    tree_compact_kernel<<<grid, block, 0, s>>>(mask, mask_stride, req_to_token, req_stride,
                                               prefix_lens, width, num_rows, num_actual_rows,
                                               page_table, table_stride, seqlens);
    return (int)hipGetLastError();
}

}  // namespace mla
