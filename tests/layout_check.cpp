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
void check_pv_split() {
    using S = PvSplitAddr<KV8>;
    for (int lane = 0; lane < 64; ++lane)
        for (int w = 0; w < 4; ++w)
            for (int md = 0; md < S::kBlocksPerWave; ++md)
                for (int kk = 0; kk < 2; ++kk)
                    for (int hi = 0; hi < (KV8 ? 1 : 2); ++hi) {
                        const int ref = S::reference(lane, w, md, kk, hi);
                        const int dec = S::decomposed(lane, w, md, kk, hi);
                        CHECK(ref == dec, "pv split kv8=%d lane=%d w=%d md=%d kk=%d hi=%d", KV8, lane, w, md, kk, hi);
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
    check_score<32, false>();
    check_score<32, true>();
    check_score<16, false>();
    check_score<16, true>();
    check_pv<32, false>();
    check_pv<32, true>();
    check_pv<16, false>();
    check_pv<16, true>();
    check_pv_split<false>();
    check_pv_split<true>();
    check_pbuf();
    if (failures) {
        std::printf("FAILED: %d\n", failures);
        return 1;
    }
    std::printf("layout ok\n");
    return 0;
}
