// Host check of the decode tile layout (paged_mla_decode_amd/csrc/mla_tile_layout.h):
//  1. the direct-to-LDS load mapping covers every (token, chunk) of a tile once;
//  2. every decomposed LDS read address (base register + immediate) equals the
//     plain chunk_offset() formula, for every lane and every instance;
//  3. the transposed reads of a 16-lane group cover a contiguous 4x16 (bf16) or
//     8x16 (fp8) block, as the hardware instruction requires.
#include <cstdio>
#include <set>
#include <utility>
#include <vector>

#include "mla_tile_layout.h"

using namespace mla;
static int failures = 0;
#define CHECK(c, ...) do { if (!(c)) { if (failures < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } ++failures; } } while (0)

template <bool KV8>
void check_dma() {
    using L = TileLayout<KV8>;
    std::set<std::pair<int, int>> seen;
    for (int b = 0; b < L::kNB; ++b) {
        const int tb = b % L::kNTB, cg = b / L::kNTB;
        for (int lane = 0; lane < 64; ++lane) {
            const int t = L::block_token(tb, lane), j = L::block_chunk(cg, lane);
            CHECK(t >= 0 && t < L::kTile && j >= 0 && j < L::kCPT, "dma out of tile kv8=%d", KV8);
            CHECK(L::chunk_offset(t, j) == b * 1024 + lane * 16, "dma slot mismatch kv8=%d b=%d lane=%d", KV8, b, lane);
            CHECK(seen.insert({t, j}).second, "dma duplicate kv8=%d", KV8);
        }
    }
    CHECK((int)seen.size() == L::kTile * L::kCPT, "dma coverage kv8=%d", KV8);
}

// The kernels issue load i of wave w (block b = w + HS i) as a per-row base
// plus a compile-time byte offset: with one token row per wave (HS a multiple
// of kNTB) the chunk group is w / kNTB + (HS / kNTB) i; with kKs = kNTB / HS
// rows, row k = i % kKs is token block w + HS k and the chunk group is i / kKs.
template <bool KV8>
void check_dma_immediates(int HS) {
    using L = TileLayout<KV8>;
    const int kKs = HS >= L::kNTB ? 1 : L::kNTB / HS;
    for (int w = 0; w < HS; ++w)
        for (int i = 0; w + HS * i < L::kNB; ++i) {
            const int b = w + HS * i;
            const int tb_expect = kKs == 1 ? w % L::kNTB : w + HS * (i % kKs);
            const int cg_expect = kKs == 1 ? w / L::kNTB + (HS / L::kNTB) * i : i / kKs;
            CHECK(b % L::kNTB == tb_expect, "dma imm token block kv8=%d HS=%d w=%d i=%d", KV8, HS, w, i);
            CHECK(b / L::kNTB == cg_expect, "dma imm chunk group kv8=%d HS=%d w=%d i=%d", KV8, HS, w, i);
            const int off = (kKs == 1 ? (HS / L::kNTB) * i : i / kKs) * L::kCG * 16;
            CHECK(off >= 0 && off < 4096, "dma imm offset range");
        }
}

template <int HW, bool KV8>
void check_score() {
    using S = ScoreAddr<HW, KV8>;
    for (int lane = 0; lane < 64; ++lane)
        for (int blk = 0; blk < S::kBlocks; ++blk)
            for (int s = 0; s < S::kSteps; ++s) {
                const int ref = S::reference(lane, s, blk);
                const int dec = S::base(lane, S::base_index(s, blk)) + S::delta(s);
                CHECK(ref == dec, "score hw=%d kv8=%d lane=%d s=%d blk=%d ref=%d dec=%d", HW, KV8, lane, s, blk, ref, dec);
                CHECK(ref >= 0 && ref < TileLayout<KV8>::kTileBytes, "score out of tile");
            }
    // Each 32-token tile: every (token, k-chunk) pair is read by exactly one lane per step.
    for (int s = 0; s < S::kSteps; ++s) {
        std::set<int> offs;
        for (int blk = 0; blk < S::kBlocks; ++blk)
            for (int lane = 0; lane < 64; ++lane) offs.insert(S::reference(lane, s, blk));
        CHECK((int)offs.size() == 64 * S::kBlocks, "score step %d reads overlap hw=%d kv8=%d", s, HW, KV8);
    }
}

template <int HW, bool KV8>
void check_pv() {
    using P = PvAddr<HW, KV8>;
    using L = TileLayout<KV8>;
    const int kks = HW == 32 ? 2 : 1;
    for (int lane = 0; lane < 64; ++lane)
        for (int md = 0; md < P::kDBlocks; ++md)
            for (int kk = 0; kk < kks; ++kk)
                for (int hi = 0; hi < P::kHalves; ++hi) {
                    const int ref = P::reference(lane, md, kk, hi);
                    const int dec = P::base(lane, P::base_index(md)) + P::delta(md, kk, hi);
                    CHECK(ref == dec, "pv hw=%d kv8=%d lane=%d md=%d kk=%d hi=%d ref=%d dec=%d", HW, KV8, lane, md, kk, hi, ref, dec);
                    CHECK(ref >= 0 && ref + 8 <= L::kTileBytes, "pv out of tile");
                    CHECK(ref % 8 == 0, "pv read not 8-byte aligned");
                }
}

template <bool KV8>
void check_h128() {
    using L = H128Layout<KV8>;
    // direct loads cover every (token, chunk) of a tile once, in lane order within a block
    std::set<std::pair<int, int>> seen;
    for (int b = 0; b < L::kNB; ++b) {
        const int tb = b % L::kNTB, cg = b / L::kNTB;
        for (int lane = 0; lane < 64; ++lane) {
            const int t = L::block_token(tb, lane), j = L::block_chunk(cg, tb, lane);
            CHECK(t >= 0 && t < L::kTile && j >= 0 && j < L::kCPT, "h128 dma out of tile kv8=%d", KV8);
            CHECK(L::chunk_offset(t, j) == b * 1024 + lane * 16, "h128 dma slot kv8=%d b=%d lane=%d", KV8, b, lane);
            CHECK(L::block_chunk(cg, tb, lane) == L::block_chunk(0, tb, lane) + cg * L::kCG, "h128 dma chunk group");
            CHECK(seen.insert({t, j}).second, "h128 dma duplicate kv8=%d", KV8);
        }
    }
    CHECK((int)seen.size() == L::kTile * L::kCPT, "h128 dma coverage kv8=%d", KV8);
    // score reads: decomposition, coverage, and one 16-byte bank group per lane of each 16-lane pass
    std::set<int> all;
    for (int s = 0; s < L::kScoreReads; ++s) {
        for (int lane = 0; lane < 64; ++lane) {
            const int ref = L::score_ref(lane, s);
            CHECK(ref == L::score_ref(lane, L::score_base_index(s)) + L::score_delta(s),
                  "h128 score kv8=%d lane=%d s=%d", KV8, lane, s);
            CHECK(ref % 16 == 0 && ref >= 0 && ref + 16 <= L::kTileBytes, "h128 score range");
            CHECK(all.insert(ref).second, "h128 score overlap");
        }
        for (int p = 0; p < 4; ++p) {
            std::set<int> banks;
            for (int lane = 16 * p; lane < 16 * p + 16; ++lane) banks.insert((L::score_ref(lane, s) / 16) % 16);
            CHECK(banks.size() == 16, "h128 score bank conflict kv8=%d s=%d pass=%d (%zu groups)", KV8, s, p, banks.size());
        }
    }
    CHECK((int)all.size() == L::kTileBytes / 16, "h128 score coverage");
    // query feature order: every feature once per lane group pair
    std::set<int> feats;
    for (int u = 0; u < 36; ++u)
        for (int g = 0; g < 2; ++g) {
            const int f = L::q_feature(u, g);
            CHECK(f % 8 == 0 && f < 576 && (f < 512) == (u < 32), "h128 q feature");
            CHECK(feats.insert(f).second, "h128 q feature duplicate");
            // the features lane group g of k-slice u multiplies are the ones it reads
            const int gran = KV8 ? 2 * (u / 2) + g : 2 * u + g;
            const int byte0 = KV8 ? 8 * (u % 2) : 0;
            CHECK(f == (KV8 ? 16 * gran + byte0 : 8 * gran), "h128 q feature vs granule");
        }
    // P . latent reads: decomposition and the general kernel's addressing of the same block
    using P = PvAddr<32, KV8>;
    std::set<int> cols;
    for (int lane = 0; lane < 64; ++lane)
        for (int w = 0; w < 4; ++w)
            for (int md = 0; md < 4; ++md) {
                for (int kk = 0; kk < 2; ++kk)
                    for (int hi = 0; hi < L::kPvBases; ++hi) {
                        const int ref = L::pv_ref(lane, 4 * md + w, kk, hi);
                        CHECK(ref == L::pv_base(lane, w, hi) + L::pv_delta(md, kk),
                              "h128 pv kv8=%d lane=%d w=%d md=%d kk=%d hi=%d", KV8, lane, w, md, kk, hi);
                        CHECK(ref >= 0 && ref + 8 <= L::kTileBytes && ref % 8 == 0, "h128 pv range");
                        // same (token, column) as the general layout's read of this block
                        const int gref = P::reference(lane, 4 * md + w, kk, hi);
                        const int gt = (gref / 1024) % L::kNTB * L::kTPB + (gref % 1024) / (16 * L::kCG);
                        const int lt = (ref / 1024) % L::kNTB * L::kTPB + (ref % 1024) / (16 * L::kCG);
                        CHECK(gt == lt && gref / 1024 == ref / 1024 && gref % 16 == ref % 16, "h128 pv element");
                    }
                for (int r = 0; r < 16; ++r) {
                    const int c = L::column(w, md, lane / 32, r);
                    CHECK(c == 32 * (4 * md + w) + 8 * (r / 4) + 4 * (lane / 32) + r % 4, "h128 column");
                    cols.insert(c);
                }
            }
    CHECK(cols.size() == 512, "h128 columns cover the latent: %zu", cols.size());
    // transposed reads: the 8-byte pieces of each 32-lane pass fill the 64 banks
    for (int blk = 0; blk < 16; ++blk)
        for (int kk = 0; kk < 2; ++kk)
            for (int hi = 0; hi < L::kPvBases; ++hi)
                for (int p = 0; p < 2; ++p) {
                    std::set<int> pairs;
                    for (int lane = 32 * p; lane < 32 * p + 32; ++lane) pairs.insert((L::pv_ref(lane, blk, kk, hi) / 8) % 32);
                    CHECK(pairs.size() == 32, "h128 pv bank conflict kv8=%d blk=%d kk=%d hi=%d pass=%d (%zu)", KV8, blk, kk,
                          hi, p, pairs.size());
                }
}

void check_out_stage() {
    // Round md: wave w, lane group g, value group r4 writes 16 bytes at
    // (head, 32 w + 8 r4 + 4 g); the store pass reads 16-byte units row-major.
    std::set<int> offs;
    for (int h = 0; h < 128; ++h)
        for (int c = 0; c < 128; c += 4) {
            const int o = OutStage::offset(h, c);
            CHECK(o % 16 == 0 && o + 16 <= OutStage::kBytes, "out stage offset");
            CHECK(offs.insert(o).second, "out stage overlap");
        }
    std::set<int> banks;
    for (int h = 0; h < 16; ++h) banks.insert((OutStage::offset(h, 36) / 16) % 16);
    CHECK(banks.size() == 16, "out stage bank spread %zu", banks.size());
}

template <int R>
void check_out_stage_bf16() {
    using S = OutStageBf16<R>;
    // store pass: 16-byte units of 8 columns, row-major, every unit once
    std::set<int> offs;
    for (int h = 0; h < 128; ++h)
        for (int c = 0; c < S::kCols; c += 8) {
            const int o = S::offset(h, c);
            CHECK(o % 16 == 0 && o + 16 <= S::kBytes, "bf16 out stage offset R=%d", R);
            CHECK(offs.insert(o).second, "bf16 out stage overlap R=%d", R);
        }
    // write pass: 32 heads at one column, 8 bytes each, at most two per 8-byte bank pair
    for (int c = 0; c < S::kCols; c += 4) {
        int count[32] = {};
        for (int h = 0; h < 32; ++h) ++count[(S::offset(h, c) / 8) % 32];
        for (int b = 0; b < 32; ++b) CHECK(count[b] <= 2, "bf16 out stage write conflicts R=%d col=%d", R, c);
    }
}

void check_pbuf() {
    std::set<int> offs;
    for (int h = 0; h < 128; ++h)
        for (int kk = 0; kk < 2; ++kk)
            for (int g = 0; g < 2; ++g) {
                const int o = PBuf::offset(h, kk, g);
                CHECK(o % 16 == 0 && o + 16 <= PBuf::kBytes, "pbuf offset");
                CHECK(offs.insert(o).second, "pbuf overlap");
            }
    // 16 consecutive heads at the same token chunk start on 16 distinct 4-bank groups.
    std::set<int> banks;
    for (int h = 0; h < 16; ++h) banks.insert((PBuf::offset(h, 0, 0) / 4) % 64 / 4);
    CHECK(banks.size() == 16, "pbuf bank spread %zu", banks.size());
}

int main() {
    check_dma<false>();
    check_dma<true>();
    for (int HS : {2, 4}) {
        check_dma_immediates<false>(HS);
        check_dma_immediates<true>(HS);
    }
    check_score<32, false>();
    check_score<32, true>();
    check_score<16, false>();
    check_score<16, true>();
    check_pv<32, false>();
    check_pv<32, true>();
    check_pv<16, false>();
    check_pv<16, true>();
    check_h128<false>();
    check_h128<true>();
    check_pbuf();
    check_out_stage();
    check_out_stage_bf16<1>();
    check_out_stage_bf16<2>();
    if (failures) {
        std::printf("FAILED: %d\n", failures);
        return 1;
    }
    std::printf("layout ok\n");
    return 0;
}
