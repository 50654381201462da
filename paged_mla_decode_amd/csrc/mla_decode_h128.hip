// gfx950 decode kernel for 128 query heads (DeepSeek-V2/V3 shapes).
//
// One workgroup of 4 waves (one per SIMD) per CU, persistent: it runs the
// plan's list of work items for it (an item is a query row and a token chunk).
// Per 32-token tile:
//   * Score: wave w computes S^T = C . Q^T for heads 32w .. 32w+31 on the
//     32x32x16 bf16 MFMA; its absorbed query (144 VGPRs) stays in registers.
//   * Softmax against a fixed per-head reference (the chunk's first-tile max),
//     so that the sums and outputs never need rescaling (an exact rerun covers
//     score spreads beyond 2^64).
//   * The bf16 probabilities of all 128 heads go through a 10 KiB LDS buffer.
//   * P . latent is split by latent columns: wave w computes O for all 128
//     heads over latent blocks 4 md + w (md = 0..3). Every latent element goes
//     through the (slow) LDS transpose read once per workgroup instead of once
//     per wave; the probabilities are read back with plain 16-byte reads.
//
// Iteration j computes the score of tile j and the P . latent product of tile
// j-1. The score MFMAs are spread between the product MFMAs (the score's LDS
// reads, every wave reading the whole tile, then run under matrix-core work),
// and the softmax of tile j rides between the last products: one wave per SIMD
// has no other wave to hide its LDS waits or VALU work behind. The MFMAs are
// volatile inline assembly so that this order holds.
//
// Memory pipeline. Tiles stream HBM -> LDS through a ring of kStages buffers
// with direct 16-byte loads (tiles j+1 .. j+kStages-2 in flight while j and
// j-1 are computed). The page-table entries of a tile travel the same queue,
// kStages - 2 iterations ahead of its data, into a small LDS ring: when the
// data loads of a tile are issued, an earlier wait has already covered its
// entries. The loop therefore has no scalar memory loads in flight while it
// waits on LDS reads (the compiler would make every LDS wait a full wait on
// them), and no load of its own the compiler could wait on. Where every tile
// lies in one page (PT), a tile's page number is one scalar load at the top of
// the iteration, consumed before the iteration's first LDS read.
//
// Output. After the last tile, the normalised outputs go through LDS (bf16:
// all 512 columns at once where the ring holds them; fp32: four rounds of 128
// columns), so that every store instruction writes whole head rows.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "mla_append.h"
#include "mla_device.h"
#include "mla_internal.h"
#include "mla_tile_layout.h"

namespace mla {
namespace {
using namespace dev;

// Tile ring depth: LDS holds kStages tiles, the probability buffer (two for
// the fp32-output mode) and the page-index ring, within 160 KiB.
template <bool KV8, bool OUT32>
struct H128Stages {
    static constexpr int value = KV8 ? 6 : (OUT32 ? 3 : 4);
};

// Wait states between the last inline-assembly MFMAs that accumulate into the
// 16 output accumulators and the VALU accesses that follow (see settle_v). One
// statement ties all 16, so no access can be scheduled before it.
__device__ __forceinline__ void settle_o(f32x16 (&O)[4][4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(O[0][0]), "+a"(O[0][1]), "+a"(O[0][2]), "+a"(O[0][3]), "+a"(O[1][0]), "+a"(O[1][1]),
                   "+a"(O[1][2]), "+a"(O[1][3]), "+a"(O[2][0]), "+a"(O[2][1]), "+a"(O[2][2]), "+a"(O[2][3]),
                   "+a"(O[3][0]), "+a"(O[3][1]), "+a"(O[3][2]), "+a"(O[3][3]));
}

// QF8: the fp8 score (e4m3fn cache, bf16 output, plain decode). The query
// comes as e4m3fn codes and a per-head exponent (quantize_query_kernel); the
// score runs on the 32x32x64 fp8 MFMA, whose operands are the tile's fp8 bytes
// as read, with no widening.
// NT: the tile loads carry the non-temporal hint (DecodeArgs::stream_tiles; a
// parameter of its own, since a branch between the two forms in the loop cost
// most of what the hint gains).
// PT: every tile lies in one page (page size a power of two of at least 32
// tokens; chunks start on tile boundaries), plain and append decodes. A tile's page number
// is one scalar load and its address a wave-uniform base plus a fixed per-lane
// offset, instead of per-lane page indices staged through LDS.
template <bool KV8, bool OUT32, int MODE, bool QF8 = false, bool NT = false, bool PT = false>
__global__ __launch_bounds__(256) void decode_h128_kernel(const DecodeArgs a) {
    static_assert(!QF8 || (KV8 && !OUT32 && MODE == kModePlain), "fp8 score: fp8 cache, bf16 output, plain decode");
    static_assert(!NT || !KV8, "the hint is for bf16 tiles");
    static_assert(!PT || MODE == kModePlain || MODE == kModeAppend, "page-uniform tiles: plain and append decodes");
    constexpr int HS = 4;
    using L = H128Layout<KV8>;
    constexpr int kLoadsMax = (L::kNB + HS - 1) / HS;
    constexpr int kLoadsMin = L::kNB / HS;
    constexpr int kSteps = 36;  // MFMA k-slices of 16 over the 576 features
    constexpr int kDW = 4;      // output blocks per wave
    constexpr int kStages = H128Stages<KV8, OUT32>::value;
    constexpr int kAhead = kStages - 2;         // iteration j issues the data of tile j + kAhead
    constexpr int kIdxAhead = 2 * kStages - 4;  // ... and the page indices of tile j + kIdxAhead
    constexpr int kPipe = 4;
    static_assert(HS >= L::kNTB, "one token per lane per tile");
    static_assert(kStages >= 3, "tiles j-1 and j are in use while j+1 loads");
    static_assert(kAhead * (kLoadsMax + 1) < 64, "vmcnt budget");
    static_assert(OutStage::kBytes <= kStages * L::kTileBytes, "output staging reuses the tile ring");
    // bf16 output: one staging round if the tile ring holds all 512 columns.
    constexpr int kOutRounds = OutStageBf16<1>::kBytes <= kStages * L::kTileBytes ? 1 : 2;
    using OS = OutStageBf16<kOutRounds>;
    static_assert(OUT32 || OS::kBytes <= kStages * L::kTileBytes, "bf16 output staging reuses the tile ring");
    __shared__ __attribute__((aligned(1024))) char smem[kStages * L::kTileBytes];
    __shared__ __attribute__((aligned(16))) char pbuf[(OUT32 ? 2 : 1) * PBuf::kBytes];
    __shared__ __attribute__((aligned(16))) int idx_ring[kStages][HS][64];
    __shared__ float l_sh[128];
    __shared__ float wa_sh[128], wb_sh[128];  // fused prefix merge: per-head weights
    __shared__ int rerun_flag[HS];

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Persistent worker: the plan's items [workers[w], workers[w+1]) in order.
    const int item_end = a.workers[blockIdx.x + 1];
    // The bf16 query, held across items: the last iteration of an item (which
    // only finishes the P . latent product) loads the next item's query, so that
    // its transfer overlaps that product and the output stage (q_ready).
    bf16x8 q[QF8 ? 1 : kSteps];
    bool q_ready = false;
    for (int item = a.workers[blockIdx.x]; item < item_end; ++item) {
        // The thread index passes through an empty asm so that every per-lane
        // address is computed anew for each item: hoisted out of the item loop
        // they would be held across it, spilled, and reloaded behind waits that
        // also drain the output stores in flight.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const mla_work_item it = a.items[item];
        const int ps = a.page_size;
        const int kv_begin = it.kv_begin;
        int kv_end = it.kv_end;
        if (a.kv_lens) kv_end = min(kv_end, a.kv_lens[it.request]);
        // Single-pass tree verify: the row's last chunk ends with its suffix
        // slots, tokens [lb, lb + visible) read from its row of the table.
        int lb = kv_end;
        const int32_t* sfx_row = nullptr;
        if (MODE == kModeTree && __builtin_amdgcn_readfirstlane(it.flags) & MLA_ITEM_LAST_CHUNK) {
            // Wave-uniform values, kept in scalar registers.
            const int row = __builtin_amdgcn_readfirstlane(it.row);
            lb = __builtin_amdgcn_readfirstlane(it.kv_end) - a.sfx_max;
            kv_end = lb + min(max(a.sfx_lens[row], 0), a.sfx_max);
            sfx_row = a.sfx_table + (int64_t)row * a.sfx_stride;
        }
        const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + kTile - 1) / kTile : 0;
        const int hq = lane & 31, gq = lane >> 5;
        const int head = it.head_begin + 32 * w + hq;  // this lane's head in the score phase
        // The bf16 query of this lane's head in query row `row`: 36 k-slices of 8 features.
        auto load_query = [&](int row) {
            const uint16_t* qn = a.q_nope + (int64_t)row * a.qn_sn + (int64_t)head * a.qn_sh;
            const uint16_t* qr = a.q_rope + (int64_t)row * a.qr_sn + (int64_t)head * a.qr_sh;
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int f = L::q_feature(u, gq);
                q[u] = u < 32 ? load_bf16x8(qn + f) : load_bf16x8(qr + (f - kLatent));
            }
        };

        // ---- tile loads ----
        // Wave w loads token block tb of every tile (kLoads 1 KiB blocks). Its
        // page-index slot holds the page of each of those tokens (tail tokens are
        // clamped to the last valid one, so no load leaves the request's pages).
        const int tb = w % L::kNTB;
        const int32_t* page_table = a.kv_indices + it.page_base;
        const int dma_lane_off = L::block_chunk(0, tb, lane) * 16;
        auto page_of = [&](int tok) { return a.page_shift >= 0 ? tok >> a.page_shift : tok / ps; };
        auto issue_idx = [&](int tile, int slot) {
            const int tok = min(kv_begin + tile * kTile + tb * L::kTPB + min(lane, L::kTPB - 1), kv_end - 1);
            const int32_t* src = page_table + page_of(tok);
            if (MODE == kModeTree && tok >= lb) src = sfx_row + (tok - lb);
            dma4(src, (LDS_AS int*)&idx_ring[slot][w][0]);
        };
        // A tile's loads: the address of this lane's 16 bytes in load 0 and
        // this wave's LDS base, then the loads themselves (issue_load<i>).
        // Load i of this wave is block b = w + HS i, chunk group
        // b / kNTB = w / kNTB + (HS / kNTB) i: a per-wave base plus 128 i bytes
        // in the row (both layouts), and 1 KiB block b in LDS.
        static_assert(HS % L::kNTB == 0 && (HS / L::kNTB) * L::kCG * 16 == 128, "immediate step");
        struct TileAddr {
            const uint8_t* rowp;  // PT: the wave-uniform base
            uint32_t lds0;
            uint32_t off;  // PT: this lane's offset from rowp
        };
        auto tile_addr = [&](int tile, int slot) {
            if constexpr (PT) {
                // The tile's tokens [t0, t0 + 32) share page t0 >> page_shift; tail
                // tokens are clamped to the last valid one, as below, and a tile
                // past the chunk (never issued) to the last tile.
                const int t0 = kv_begin + min(tile, ntiles - 1) * kTile;
                const int page = ((const __attribute__((address_space(4))) int32_t*)page_table)[t0 >> a.page_shift];
                const int tok = min(L::block_token(tb, lane), kv_end - 1 - t0);
                return TileAddr{a.cache + ((int64_t)page * ps + (t0 & (ps - 1))) * L::kRowBytes + (w / L::kNTB) * L::kCG * 16,
                                (uint32_t)(uintptr_t)((LDS_AS char*)smem + slot * L::kTileBytes + w * 1024),
                                (uint32_t)(tok * L::kRowBytes + dma_lane_off)};
            }
            const int tau = min(kv_begin + tile * kTile + L::block_token(tb, lane), kv_end - 1);
            const int page = idx_ring[slot][w][lane / L::kCG];
            const int row = a.page_shift >= 0 ? (tau & (ps - 1)) : tau % ps;
            return TileAddr{a.cache + ((int64_t)page * ps + row) * L::kRowBytes + dma_lane_off + (w / L::kNTB) * L::kCG * 16,
                            (uint32_t)(uintptr_t)((LDS_AS char*)smem + slot * L::kTileBytes + w * 1024), 0u};
        };
        auto issue_load = [&](auto ic, const TileAddr& t, auto nt_c) {
            constexpr int i = decltype(ic)::value;
            if (L::kNB % HS == 0 || w + HS * i < L::kNB) {
                if constexpr (PT)
                    dma16_imm_s<128 * i, 1024 * HS * i, decltype(nt_c)::value>(t.rowp, t.off, t.lds0);
                else
                    dma16_imm<128 * i, 1024 * HS * i, decltype(nt_c)::value>(t.rowp, t.lds0);
            }
        };
        auto issue_tile = [&](int tile, int slot) {
            const TileAddr t = tile_addr(tile, slot);
            [&]<int... I>(std::integer_sequence<int, I...>) {
                (issue_load(std::integral_constant<int, I>{}, t, std::bool_constant<NT>{}), ...);
            }(std::make_integer_sequence<int, kLoadsMax>{});
        };
        auto wrap = [](int x) { return x >= kStages ? x - kStages : x; };
        // Tile t and its page indices live in slot t % kStages.
        auto prologue_idx = [&] {
            if constexpr (!PT) {
#pragma unroll
                for (int t = 0; t < kAhead; ++t)
                    if (t < ntiles) issue_idx(t, t);
            }
        };
        // The first tiles: the product at j = 0 reads slot kStages-1 (first
        // loaded at j = 1) and the probability buffer, both zeroed; then the data
        // of tiles 0 .. kAhead-1, each preceded by the page indices of the tile
        // kAhead later (as iteration t - kAhead would).
        auto start_tiles = [&] {
            {
                using V4 = __attribute__((__vector_size__(4 * sizeof(int)))) int;
                LDS_AS V4* z = (LDS_AS V4*)(smem + (kStages - 1) * L::kTileBytes);
                for (int k = tid; k < L::kTileBytes / 16; k += 256) z[k] = V4{0, 0, 0, 0};
                LDS_AS V4* zp = (LDS_AS V4*)pbuf;
                for (int k = tid; k < (OUT32 ? 2 : 1) * PBuf::kBytes / 16; k += 256) zp[k] = V4{0, 0, 0, 0};
            }
#pragma unroll
            for (int t = 0; t < kAhead; ++t) {
                if (!PT && t + kAhead < ntiles) issue_idx(t + kAhead, wrap(t + kAhead));
                if (t < ntiles) issue_tile(t, t);
            }
        };
        // ---- page indices of the first tiles, the absorbed query, the first tiles ----
        // The query loads go out right behind the page indices, and the first wait
        // leaves them in flight (loads retire in issue order, so vmcnt <= kQLoads
        // means the indices have landed): the query's transfer overlaps the
        // indices' round trip. The first tiles follow, and one wait covers them
        // and the query.
        // bf16: 36 k-slices of 8 features. fp8 score: 9 steps of 32 codes, the
        // features 64 v + 16 gq + [0, 16) and 64 v + 32 + 16 gq + [0, 16), which
        // are the bytes the step's two tile reads give this lane, and the head's
        // exponent (19 loads).
        constexpr int kQLoads = kSteps;  // the bf16 query's vector loads
        prologue_idx();
        u32x8 q8[QF8 ? 9 : 1];
        int q8e = 0;
        if constexpr (QF8) {
            const int64_t qrow = (int64_t)it.row * a.num_heads + head;
            const uint8_t* src = a.q8 + qrow * kRow + 16 * gq;
#pragma unroll
            for (int v = 0; v < 9; ++v) {
                const u32x4 lo = *reinterpret_cast<const u32x4*>(src + 64 * v);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 64 * v + 32);
                q8[v] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            q8e = a.q8_exp[qrow];
        } else if (!q_ready) {
            load_query(it.row);
        }
        // The page indices: the bf16 query is 36 vector loads issued after them,
        // which the wait leaves in flight (tests/test_isa_waits.py checks the
        // compiled kernels for at least kQLoads loads between the last index load
        // and this wait). The fp8-score instantiation waits for everything: its
        // query loads share the stretch with spill traffic the compiler places.
        if constexpr (PT) {
            // No page indices to wait for: the tiles go out behind the query.
        } else if (QF8 || q_ready) {
            wait_vmcnt<0>();  // (a prefetched query went out long before the indices)
        } else {
            wait_vmcnt_query<kQLoads>();
        }
        q_ready = false;
        if (MODE == kModeAppend && __builtin_amdgcn_readfirstlane(it.flags) & MLA_ITEM_LAST_CHUNK) {
            // Fused append: the request's new row goes to the cache before any
            // wave loads a tile that holds it.
            append_row<KV8>(a, it, tid, 256);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the row's stores are done
            __syncthreads();
        }
        if (ntiles > 0) start_tiles();
        // vmcnt(0), as a builtin the compiler accounts for: the query and the first
        // tiles have landed, so the compiler places no waits of its own in the
        // loop, where they would also drain the tiles in flight.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // Score scale (log2 units), times 2^e for the fp8 score.
        const float sl2 = QF8 ? ldexpf(a.scale_log2, q8e) : a.scale_log2;

        int sbase[L::kScoreBases], pbase[L::kPvBases];
#pragma unroll
        for (int i = 0; i < L::kScoreBases; ++i) sbase[i] = L::score_ref(lane, i);
#pragma unroll
        for (int i = 0; i < L::kPvBases; ++i) pbase[i] = L::pv_base(lane, w, i);
        const int p_wr = PBuf::offset(32 * w + hq, 0, gq);  // this lane's probabilities, kk = 0
        const int p_rd = PBuf::offset(hq, 0, gq);           // head block hb adds hb * 32 rows

        f32x16 O[kDW][4];
        float m_ref = -INFINITY, m_true = -INFINITY;
        float l_part = 0.f;

        for (int pass = 0; pass < 2; ++pass) {
            {
                // Zeroed by the matrix core: a VALU zeroing of 256 AGPRs makes the
                // compiler spill a zero vector and wait on its reload here.
                const bf16x8 z = {};
#pragma unroll
                for (int i = 0; i < kDW; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mfma32_zero_a(O[i][j], z);
            }
            l_part = 0.f;

            if (ntiles > 0) {
                if (pass > 0) {
                    prologue_idx();
                    wait_vmcnt_barrier<0>();
                    start_tiles();
                }
                // Iterations j = 0 .. ntiles - 1 run one body: the score of tile j
                // (slot cur) and the P . latent product of tile j-1 (slot prv). At
                // j = 0 the product reads a zeroed slot and a zeroed probability
                // buffer and adds exact zeros. The last iteration (kLast, j = ntiles)
                // only finishes the product of tile ntiles - 1. With an fp8 cache and
                // in the tree-verify pass it loads the next item's query meanwhile,
                // unless this item reruns (every wave's rerun flag is written at the
                // end of iteration ntiles - 1): skewed fp8 69.0 -> 66.7 us, tree
                // verify 534 -> 529 us per call. The bf16 decode measured 1-2% slower
                // with it (V3) and loads each query at its item's start.
                constexpr bool kPrefetchQ = !QF8 && (KV8 || MODE == kModeTree);
                auto iteration = [&](auto last_c, int j, int cur) {
                    constexpr bool kLast = decltype(last_c)::value;
                    const int prv = cur == 0 ? kStages - 1 : cur - 1;
                    // Tile j has landed; every wave is past iteration j-1, so P(j-1)
                    // is visible and the slot of tile j-2 is free.
                    if constexpr (!kLast)
                        wait_tiles_barrier<kStages - 3, kLoadsMin>(min(kStages - 3, ntiles - 1 - j));
                    else
                        lds_barrier();
                    if constexpr (kLast && kPrefetchQ) {
                        int any = 0;
#pragma unroll
                        for (int k = 0; k < HS; ++k) any |= rerun_flag[k];
                        if (!any && item + 1 < item_end) {
                            load_query(a.items[item + 1].row);
                            q_ready = true;
                        }
                    }
                    if (!PT && !kLast && j + kIdxAhead < ntiles) issue_idx(j + kIdxAhead, wrap(cur + kIdxAhead % kStages));
                    // The data of tile j + kAhead. Issuing a tile's loads stalls each
                    // wave about 550 cycles (per-phase timestamps, V3). With an fp8
                    // cache they go out spread between this iteration's MFMAs below
                    // (skewed fp8: 74 -> 70 us per call); with bf16 the spread was
                    // slower (V3: 134.5 -> 137 us) and they go out here, together.
                    constexpr bool kSpreadLoads = KV8;
                    const bool do_dma = !kLast && j + kAhead < ntiles;
                    TileAddr dma{};
                    if (do_dma) {
                        if constexpr (kSpreadLoads)
                            dma = tile_addr(j + kAhead, wrap(cur + kAhead));
                        else
                            issue_tile(j + kAhead, wrap(cur + kAhead));
                    }

                    const LDS_AS char* Ts = (const LDS_AS char*)smem + cur * L::kTileBytes;
                    const LDS_AS char* Tp = (const LDS_AS char*)smem + prv * L::kTileBytes;
                    const LDS_AS char* Pb = (const LDS_AS char*)pbuf;

                    // Score operand s (one or two k-slices): raw tile bytes; fp8 codes
                    // are widened to bf16 next to their MFMA. The bf16 operands of both
                    // products come from LDS and the query from global memory, so their
                    // MFMAs skip the wait states a VALU-written operand needs (<KV8>).
                    using SOp = std::conditional_t<KV8, u32x4, bf16x8>;
                    auto sload = [&](int s) {
                        return *(const LDS_AS SOp*)(Ts + sbase[L::score_base_index(s)] + L::score_delta(s));
                    };
                    // Product A operand of step a = 4 kk + md (transposed reads).
                    using AOp = std::conditional_t<KV8, i32x2, i16x4[2]>;
                    struct ARaw { AOp v; };
                    auto aload = [&](int a) {
                        const int kk = a >> 2, md = a & 3;
                        ARaw r;
                        if constexpr (KV8) {
                            r.v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                (LDS_AS i32x2*)(Tp + pbase[0] + L::pv_delta(md, kk)));
                        } else {
                            r.v[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (LDS_AS i16x4*)(Tp + pbase[0] + L::pv_delta(md, kk)));
                            r.v[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (LDS_AS i16x4*)(Tp + pbase[1] + L::pv_delta(md, kk)));
                        }
                        return r;
                    };
                    auto awiden = [&](const ARaw& r) {
                        if constexpr (KV8)
                            return fp8x8_to_bf16((unsigned)r.v[0], (unsigned)r.v[1]);
                        else
                            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r.v[0], r.v[1], 0, 1, 2, 3, 4, 5, 6, 7));
                    };
                    // P(j-1) of token half kk, head block hb (B operands; lo parts for fp32 output).
                    auto pload = [&](int kk, int hb, int lo) {
                        return *(const LDS_AS bf16x8*)(Pb + lo * PBuf::kBytes + p_rd + hb * 32 * PBuf::kRow + 32 * kk);
                    };

                    // ---- schedule ----
                    // 36 score MFMAs (one accumulator chain, in VGPRs) and kPM product
                    // MFMAs (independent accumulators). The first kMix product MFMAs
                    // are spread evenly between the score MFMAs, so the score's LDS
                    // reads (each wave reads the whole tile) proceed under product
                    // MFMAs; the last kTail products carry the softmax of tile j.
                    constexpr int kSM = QF8 ? 9 : 36;
                    constexpr int kPM = OUT32 ? 64 : 32;
                    constexpr int kTail = OUT32 ? 16 : 8;
                    constexpr int kMix = kPM - kTail;
                    constexpr int kSR = L::kScoreReads;  // 36 | 18 reads
                    constexpr int kMPR = QF8 ? 1 : kSM / kSR;  // MFMAs per score read (fp8 score: 2 reads per MFMA)
                    constexpr int kPipe8 = kPipe / 2;        // fp8 score operands in flight
                    constexpr int kPPS = OUT32 ? 8 : 4;  // product MFMAs per A step

                    SOp sb[QF8 ? 1 : kPipe];
                    u32x8 sb8[QF8 ? kPipe8 : 1];
                    // fp8 score step v: tile reads 2 v and 2 v + 1 (64 features of one token).
                    auto sload8 = [&](int v) {
                        const u32x4 lo = sload(2 * v), hi = sload(2 * v + 1);
                        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    };
                    if constexpr (kLast) {
                    } else if constexpr (QF8) {
#pragma unroll
                        for (int i = 0; i < kPipe8; ++i) sb8[i] = sload8(i);
                    } else {
#pragma unroll
                        for (int i = 0; i < kPipe; ++i) sb[i] = sload(i);
                    }
                    ARaw ab[2] = {aload(0), aload(1)};
                    bf16x8 Bp[4], Bl[4];
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb) {
                        Bp[hb] = pload(0, hb, 0);
                        if (OUT32) Bl[hb] = pload(0, hb, 1);
                    }
                    f32x16 S;
                    bf16x8 Acur;

                    auto score_mfma = [&](int si) {
                        if constexpr (QF8) {
                            if (si == 0) mfma32_f8_first_v(S, sb8[0], q8[0]);
                            else mfma32_f8_acc_v(S, sb8[si % kPipe8], q8[si]);
                            if (si + kPipe8 < kSM) sb8[si % kPipe8] = sload8(si + kPipe8);
                        } else {
                            const int s = si / kMPR, h = si % kMPR;
                            bf16x8 A;
                            if constexpr (KV8) A = fp8x8_to_bf16(sb[s % kPipe][2 * h], sb[s % kPipe][2 * h + 1]);
                            else A = sb[s % kPipe];
                            if (si == 0) mfma32_first_v<KV8>(S, A, q[si]);
                            else mfma32_acc_v<KV8>(S, A, q[si]);
                            if (h == kMPR - 1 && s + kPipe < kSR) sb[s % kPipe] = sload(s + kPipe);
                        }
                    };
                    auto product_mfma = [&](int pi) {
                        const int a = pi / kPPS, hb = (pi % kPPS) / (OUT32 ? 2 : 1), lo = OUT32 ? pi % 2 : 0;
                        const int kk = a >> 2, md = a & 3;
                        if (pi % kPPS == 0) {
                            Acur = awiden(ab[a & 1]);
                            if (a + 2 < 8) ab[a & 1] = aload(a + 2);
                        }
                        const bf16x8 B = lo ? Bl[hb] : Bp[hb];
                        mfma32_acc_a<KV8>(O[md][hb], Acur, B);
                        // P of token half 1 replaces each operand after its last use in
                        // half 0.
                        if (kk == 0 && md == 3 && lo == (OUT32 ? 1 : 0)) {
                            Bp[hb] = pload(1, hb, 0);
                            if (OUT32) Bl[hb] = pload(1, hb, 1);
                        }
                    };

                    int si = 0, pi = 0;
                    if constexpr (kLast) {
#pragma unroll
                        for (int t = 0; t < kPM; ++t) product_mfma(pi++);
                        return;
                    }
                    // Slot g: a score MFMA when it advances the score's share of the
                    // slots (Bresenham spread), else a product MFMA; after every
                    // kDmaEvery-th slot one of the next tile's loads.
                    constexpr int kSlots = kSM + kMix;
                    constexpr int kDmaEvery = kSlots / kLoadsMax;
                    auto mix_slot = [&](auto gc) {
                        constexpr int g = decltype(gc)::value;
                        if constexpr ((g + 1) * kSM / kSlots != g * kSM / kSlots)
                            score_mfma(si++);
                        else
                            product_mfma(pi++);
                        if constexpr (kSpreadLoads && g % kDmaEvery == kDmaEvery / 2 && g / kDmaEvery < kLoadsMax) {
                            if (do_dma) issue_load(std::integral_constant<int, g / kDmaEvery>{}, dma, std::false_type{});
                        }
                    };
                    [&]<int... G>(std::integer_sequence<int, G...>) {
                        (mix_slot(std::integral_constant<int, G>{}), ...);
                    }(std::make_integer_sequence<int, kSlots>{});
                    settle_v(S);

                    // ---- softmax of tile j, in eight pieces between the last products ----
                    // Raw scores; the scale (positive) enters through one fma in the
                    // exponent, and the maximum of the raw scores scales to the maximum
                    // of the scaled ones. Only a tile with fewer than 32 valid tokens
                    // (the last one, and the phantom iteration) masks: value r is token
                    // 16 (r / 8) + 8 gq + r % 8.
                    const int nvalid = min(kTile, kv_end - (kv_begin + j * kTile));
                    float tmax = 0.f, ls0 = 0.f, ls1 = 0.f;
                    bf16x8 P[2], Plo[2];
                    // Each piece ends in an empty volatile statement that takes its
                    // results: volatile statements keep program order with the
                    // product MFMAs, so the piece is computed before the next one.
                    auto soft = [&](int piece) {
                        if (piece == 0) {
                            if (nvalid < kTile) {
                                const int lim = nvalid - 8 * gq;
#pragma unroll
                                for (int r = 0; r < 16; ++r)
                                    if (16 * (r >> 3) + (r & 7) >= lim) S[r] = -INFINITY;
                            }
                            asm volatile("" : "+v"(S));
                        } else if (piece == 1) {
                            tmax = fmaxf(S[0], S[1]);
#pragma unroll
                            for (int r = 2; r < 8; ++r) tmax = fmaxf(tmax, S[r]);
                            asm volatile("" : "+v"(tmax));
                        } else if (piece == 2) {
#pragma unroll
                            for (int r = 8; r < 16; ++r) tmax = fmaxf(tmax, S[r]);
                            asm volatile("" : "+v"(tmax));
                        } else if (piece == 3) {
                            tmax = max_xor32(tmax) * sl2;
                            if (j == 0 && pass == 0) m_ref = tmax;
                            m_true = fmaxf(m_true, tmax);
                            asm volatile("" : "+v"(m_ref), "+v"(m_true));
                        } else {
                            const int kk = (piece - 4) >> 1, e0 = 4 * ((piece - 4) & 1);
#pragma unroll
                            for (int e = e0; e < e0 + 4; ++e) {
                                const float pv = fast_exp2(fmaf(S[8 * kk + e], sl2, -m_ref));
                                if (e & 1)
                                    ls1 += pv;
                                else
                                    ls0 += pv;
                                P[kk][e] = (__bf16)pv;
                                if (OUT32) Plo[kk][e] = (__bf16)(pv - (float)P[kk][e]);
                            }
                            asm volatile("" : "+v"(ls0), "+v"(ls1));
                            if ((piece & 1) == 1) {
                                asm volatile("" : "+v"(P[kk]));
                                if (OUT32) asm volatile("" : "+v"(Plo[kk]));
                            }
                        }
                    };
#pragma unroll
                    for (int t = 0; t < kTail; ++t) {
                        product_mfma(pi++);
                        if (t % (kTail / 8) == kTail / 8 - 1) soft(t / (kTail / 8));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    l_part += ls0 + ls1;
                    if constexpr (kPrefetchQ) {
                        // The last tile's softmax is done: does any head need the rerun?
                        if (j == ntiles - 1) {
                            const bool over = __builtin_amdgcn_ballot_w64(m_true > m_ref + kOverflowSlack) != 0;
                            if (lane == 0) rerun_flag[w] = over ? 1 : 0;
                        }
                    }

                    // Every wave is done reading P(j-1): the buffer takes P(j).
                    lds_barrier();
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        *(LDS_AS bf16x8*)((LDS_AS char*)pbuf + p_wr + 32 * kk) = P[kk];
                        if (OUT32) *(LDS_AS bf16x8*)((LDS_AS char*)pbuf + PBuf::kBytes + p_wr + 32 * kk) = Plo[kk];
                    }
                };
                int cur = 0;
                for (int j = 0; j < ntiles; ++j) {
                    iteration(std::false_type{}, j, cur);
                    cur = wrap(cur + 1);
                }
                iteration(std::true_type{}, ntiles, cur);
                settle_o(O);
            }
            // Did any head outgrow its reference? All waves must agree (the tiles are
            // loaded cooperatively), so the flag goes through LDS.
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

        // ---- finalize ----
        const float l = sum_xor32(l_part);
        const int nh = a.num_heads;
        const float lse = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : -INFINITY;
        // Fused prefix merge of an unsplit row: out = wa * prefix + wb * this,
        // with the weights of the two states' LSE merge.
        const bool fuse = MODE == kModeMerge && it.partial < 0;
        if (gq == 0) {
            l_sh[32 * w + hq] = l;
            if (fuse) {
                const int64_t i = (int64_t)it.row * nh + head;
                const float la = a.prefix_lse[i];
                float wa = 0.f, wb = 0.f, s = -INFINITY;
                if (!(la == -INFINITY && lse == -INFINITY)) {
                    const float mx = fmaxf(la, lse);
                    const float ea = __expf(la - mx), eb = __expf(lse - mx);
                    wa = ea / (ea + eb);
                    wb = eb / (ea + eb);
                    s = mx + __logf(ea + eb);
                }
                wa_sh[32 * w + hq] = wa;
                wb_sh[32 * w + hq] = wb;
                if (a.lse) a.lse[i] = s;
            } else if (it.partial >= 0) {
                a.part_lse[(int64_t)it.partial * nh + head] = lse;
            } else if (a.lse) {
                a.lse[(int64_t)it.row * nh + head] = lse;
            }
        }
        lds_barrier();
        float inv[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            const float lh = l_sh[32 * hb + hq];
            if (MODE == kModeMerge && fuse)
                inv[hb] = lh > 0.f ? a.out_scale * wb_sh[32 * hb + hq] / lh : 0.f;
            else
                inv[hb] = lh > 0.f ? a.out_scale / lh : 0.f;
        }
        // Output rows of this item: [partial or row][head_begin + h][512].
        const int64_t row0 = (it.partial >= 0 ? (int64_t)it.partial * nh : (int64_t)it.row * nh) + it.head_begin;
        LDS_AS char* stage = (LDS_AS char*)smem;  // every wave is past its last tile read
        // Partials are stored in the output's precision.
        void* const obase = it.partial >= 0 ? a.part_out : a.out;
        if constexpr (!OUT32) {
            // bf16: [128 heads][512] in one round (two where the tile ring is
            // smaller), then every store instruction writes whole head rows with
            // 16 bytes per lane.
#pragma unroll
            for (int rd = 0; rd < kOutRounds; ++rd) {
#pragma unroll
                for (int md = rd * kDW / kOutRounds; md < (rd + 1) * kDW / kOutRounds; ++md)
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const bf16x4 v = {(__bf16)(O[md][hb][4 * r4] * inv[hb]), (__bf16)(O[md][hb][4 * r4 + 1] * inv[hb]),
                                              (__bf16)(O[md][hb][4 * r4 + 2] * inv[hb]), (__bf16)(O[md][hb][4 * r4 + 3] * inv[hb])};
                            const int col = L::column(w, md, gq, 4 * r4) - rd * OS::kCols;
                            *(LDS_AS bf16x4*)(stage + OS::offset(32 * hb + hq, col)) = v;
                        }
                lds_barrier();
                // 128 heads x kCols / 8 units of 8 columns, consecutive lanes on
                // consecutive units.
                constexpr int kUnits = OS::kCols / 8;
#pragma unroll
                for (int jj = 0; jj < 128 * kUnits / 256; ++jj) {
                    const int u = tid + 256 * jj;
                    const int h = u / kUnits, c8 = u % kUnits;
                    bf16x8 v = *(const LDS_AS bf16x8*)(stage + OS::offset(h, 8 * c8));
                    const int64_t o = (row0 + h) * kLatent + rd * OS::kCols + 8 * c8;
                    if (MODE == kModeMerge && fuse) {
                        const bf16x8 p = *(reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.prefix_out) + o));
                        const float wa = wa_sh[h];
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] + wa * (float)p[e]);
                    }
                    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(obase) + o) = v;
                }
                lds_barrier();
            }
        } else {
#pragma unroll
            for (int md = 0; md < kDW; ++md) {
#pragma unroll
                for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const f32x4 v = {O[md][hb][4 * r4] * inv[hb], O[md][hb][4 * r4 + 1] * inv[hb],
                                         O[md][hb][4 * r4 + 2] * inv[hb], O[md][hb][4 * r4 + 3] * inv[hb]};
                        const int col = L::column(w, md, gq, 4 * r4) - 128 * md;
                        *(LDS_AS f32x4*)(stage + OutStage::offset(32 * hb + hq, col)) = v;
                    }
                lds_barrier();
                // 128 heads x 32 units of 4 columns; consecutive lanes take consecutive units.
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int u = tid + 256 * j;
                    const int h = u >> 5, c4 = u & 31;
                    f32x4 v = *(const LDS_AS f32x4*)(stage + OutStage::offset(h, 4 * c4));
                    const int64_t o = (row0 + h) * kLatent + 128 * md + 4 * c4;
                    if (MODE == kModeMerge && fuse)
                        v += wa_sh[h] * *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.prefix_out) + o);
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(obase) + o) = v;
                }
                lds_barrier();
            }
        }
    }
}

}  // namespace

int launch_decode_h128(int kv_dtype, int out_dtype, const DecodeArgs& a, int num_workers, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid(num_workers), block(256);
    const bool kv8 = kv_dtype == MLA_DTYPE_FP8_E4M3FN;
    const bool o32 = out_dtype == MLA_DTYPE_FP32;
    // The fused append and the fused prefix merge are instantiations of their
    // own, so the plain decode carries none of their arguments or branches.
    const int mode = a.c_new ? kModeAppend : a.prefix_lse ? kModeMerge : a.sfx_table ? kModeTree : kModePlain;
    if (a.q8) {
        if (!kv8 || o32 || mode != kModePlain) return (int)hipErrorInvalidValue;
        if (a.page_shift >= 5)
            decode_h128_kernel<true, false, kModePlain, true, false, true><<<grid, block, 0, s>>>(a);
        else
            decode_h128_kernel<true, false, kModePlain, true><<<grid, block, 0, s>>>(a);
        return (int)hipGetLastError();
    }
    auto go = [&](auto kv8_t, auto o32_t) {
        constexpr bool K = decltype(kv8_t)::value, O = decltype(o32_t)::value;
        // The streaming hint exists for the bf16 plain and append decodes (one
        // query row per request); other modes share tiles among rows or do not
        // stream (the suffix merge reads a few slots per row).
        const bool nt = !K && a.stream_tiles;
        // Page-uniform tiles (plain and append decodes): a power-of-two page of at
        // least 32 tokens.
        const bool pt = a.page_shift >= 5;
        if (mode == kModeAppend) {
            if (nt && pt)
                decode_h128_kernel<false, O, kModeAppend, false, true, true><<<grid, block, 0, s>>>(a);
            else if (nt)
                decode_h128_kernel<false, O, kModeAppend, false, true><<<grid, block, 0, s>>>(a);
            else if (pt)
                decode_h128_kernel<K, O, kModeAppend, false, false, true><<<grid, block, 0, s>>>(a);
            else
                decode_h128_kernel<K, O, kModeAppend><<<grid, block, 0, s>>>(a);
        } else if (mode == kModeTree) {
            decode_h128_kernel<K, O, kModeTree><<<grid, block, 0, s>>>(a);
        } else if (mode == kModeMerge) {
            decode_h128_kernel<K, O, kModeMerge><<<grid, block, 0, s>>>(a);
        } else if (nt) {
            if (pt)
                decode_h128_kernel<false, O, kModePlain, false, true, true><<<grid, block, 0, s>>>(a);
            else
                decode_h128_kernel<false, O, kModePlain, false, true><<<grid, block, 0, s>>>(a);
        } else if (pt) {
            decode_h128_kernel<K, O, kModePlain, false, false, true><<<grid, block, 0, s>>>(a);
        } else {
            decode_h128_kernel<K, O, kModePlain><<<grid, block, 0, s>>>(a);
        }
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

}  // namespace mla
