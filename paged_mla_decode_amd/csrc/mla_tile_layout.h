// LDS layout of a decode tile and the per-lane address decompositions the
// decode kernel uses. Host and device code share this header: a CPU test
// checks every decomposition against chunk_offset() for every lane.
//
// A tile holds 32 cache rows (tokens). A row is split into 16-byte chunks
// (72 for bf16, 36 for fp8). The tile is stored as 1 KiB blocks, each holding
// TPB tokens x CG chunks: one direct-to-LDS load instruction of a wave writes
// its 64 lanes' 16 bytes contiguously, i.e. exactly one block. Inside a block,
// chunk c of token t sits in slot c ^ (t % CG): an XOR swizzle that spreads the
// same chunk of consecutive tokens over different LDS banks. Blocks are
// ordered chunk-group-major: block = (chunk / CG) * NTB + token / TPB.
//
// Every LDS read address of the kernel is (a per-lane base register) + (a
// compile-time immediate). The swizzle mixes lane bits and compile-time bits,
// so each read type keeps a handful of bases, one per value of the
// compile-time bits that interact with the lane bits.
#pragma once

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

template <bool KV8>
struct TileLayout {
    static constexpr int kTile = 32;
    static constexpr int kRowBytes = KV8 ? 576 : 1152;
    static constexpr int kCPT = kRowBytes / 16;  // chunks per token: 36 | 72
    static constexpr int kCG = KV8 ? 4 : 8;      // chunks per token in one block
    static constexpr int kTPB = 64 / kCG;        // tokens per block: 16 | 8
    static constexpr int kNCG = kCPT / kCG;      // chunk groups: 9
    static constexpr int kNTB = kTile / kTPB;    // token blocks: 2 | 4
    static constexpr int kNB = kNCG * kNTB;      // blocks per tile: 18 | 36
    static constexpr int kTileBytes = kNB * 1024;

    // Byte offset of chunk j of token t.
    static MLA_HD int chunk_offset(int t, int j) {
        const int b = (j / kCG) * kNTB + t / kTPB;
        return b * 1024 + ((t % kTPB) * kCG + ((j % kCG) ^ (t % kCG))) * 16;
    }
    // Which chunk lane `lane` of a block loads (the inverse swizzle), and the
    // token of the block it belongs to.
    static MLA_HD int block_token(int tb, int lane) { return tb * kTPB + lane / kCG; }
    static MLA_HD int block_chunk(int cg, int lane) {
        const int t_mod = (lane / kCG) % kCG;  // = token % CG, for every token block
        return cg * kCG + ((lane % kCG) ^ t_mod);
    }
};

// ---- Score operand (A of S^T = C . Q^T): lane reads 8 latent values of one token ----
//
// HW=32 (32x32x16 MFMA): lane holds token perm(lane % 32) and k = 16 s + 8 (lane / 32).
// The token permutation swaps bits 2 and 3, so that the accumulator rows a lane
// owns are eight consecutive tokens (what the P . latent operand needs).
// HW=16 (16x16x32 MFMA, two 16-token blocks): lane holds token
// 8 (m / 4) + m % 4 + 4 blk (m = lane % 16) and k = 32 s + 8 (lane / 16).
template <int HW, bool KV8>
struct ScoreAddr {
    using L = TileLayout<KV8>;
    static constexpr int kSteps = HW == 32 ? 36 : 18;
    static constexpr int kBlocks = HW == 32 ? 1 : 2;
    static constexpr int kBases = 4;

    static MLA_HD int token(int lane, int blk) {
        if (HW == 32) {
            const int m = lane & 31;
            return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
        }
        const int m = lane & 15;
        return 8 * (m >> 2) + (m & 3) + 4 * blk;
    }
    // Reference: byte offset of the 8 values (16 bytes bf16 / 8 bytes fp8).
    static MLA_HD int reference(int lane, int s, int blk) {
        const int g = HW == 32 ? (lane >> 5) : (lane >> 4);
        const int kbyte = (KV8 ? 1 : 2) * ((HW == 32 ? 16 : 32) * s + 8 * g);
        return L::chunk_offset(token(lane, blk), kbyte >> 4) + (kbyte & 15);
    }
    // Base index and immediate of step s of block blk.
    static MLA_HD constexpr int base_index(int s, int blk) {
        return HW == 32 ? (s % 4) : (2 * blk + (s % 2));
    }
    static MLA_HD constexpr int delta(int s) {
        return HW == 32 ? (s / 4) * (KV8 ? 2048 : 4096) : (s / 2) * (KV8 ? 2048 : 4096);
    }
    static MLA_HD int base(int lane, int bi) {
        return HW == 32 ? reference(lane, bi, 0) : reference(lane, bi % 2, bi / 2);
    }
};

// ---- P . latent operand (A of O^T = C^T . P^T): transposed LDS reads ----
//
// bf16, ds_read_b64_tr_b16: a 16-lane group reads a 4-token x 16-column block;
// lane q supplies the address of token q / 4, columns 4 (q % 4) .. +3 and
// receives column q over the 4 tokens. Two reads (hi = 0, 1) cover 8 tokens.
// fp8, ds_read_b64_tr_b8: a 16-lane group reads an 8-token x 16-byte block;
// lane q supplies token q / 2, bytes 8 (q % 2) .. +7 and receives byte column q
// over the 8 tokens.
// HW=32: output block md covers latent columns 32 md .. +31, token half kk.
// HW=16: output block md covers latent columns 16 md .. +15.
template <int HW, bool KV8>
struct PvAddr {
    using L = TileLayout<KV8>;
    static constexpr int kDBlocks = 512 / HW;
    static constexpr int kHalves = KV8 ? 1 : 2;
    static constexpr int kBases = KV8 ? (HW == 32 ? 2 : 4) : (HW == 32 ? 1 : 2);

    static MLA_HD int reference(int lane, int md, int kk, int hi) {
        const int grp = lane >> 4, q = lane & 15;
        int t, cbyte;
        if (HW == 32) {
            const int rowb = 16 * kk + 8 * (grp >> 1);
            const int colb = 32 * md + 16 * (grp & 1);  // element column
            if (KV8) {
                t = rowb + (q >> 1);
                cbyte = colb + 8 * (q & 1);
            } else {
                t = rowb + (q >> 2) + 4 * hi;
                cbyte = 2 * (colb + 4 * (q & 3));
            }
        } else {
            const int rowb = 8 * grp;
            const int colb = 16 * md;
            if (KV8) {
                t = rowb + (q >> 1);
                cbyte = colb + 8 * (q & 1);
            } else {
                t = rowb + (q >> 2) + 4 * hi;
                cbyte = 2 * (colb + 4 * (q & 3));
            }
        }
        return L::chunk_offset(t, cbyte >> 4) + (cbyte & 15);
    }
    static MLA_HD constexpr int base_index(int md) {
        return KV8 ? (HW == 32 ? (md & 1) : (md & 3)) : (HW == 32 ? 0 : (md & 1));
    }
    static MLA_HD constexpr int delta(int md, int kk, int hi) {
        if (KV8) return HW == 32 ? ((md >> 1) * 2 + kk) * 1024 : (md >> 2) * 2048;
        if (HW == 32)
            return ((md >> 1) * 4 + 2 * kk) * 1024 + hi * 512 + 64 * ((md & 1) ^ hi);
        return (md >> 2) * 4096 + hi * 512 + 64 * (((md >> 1) & 1) ^ hi);
    }
    static MLA_HD int base(int lane, int bi) {
        // The instance with delta 0 for this base.
        return reference(lane, bi, 0, 0);
    }
};

// ---- Layout of the 128-head kernel ----
// The tile geometry of TileLayout, with a swizzle chosen for that kernel's
// reads: slot = chunk ^ ((t / kTPL) % kCG), where kTPL tokens share one
// 256-byte LDS line (64 banks of 4 bytes). The sixteen lanes one pass of a
// 16-byte read serves hold sixteen consecutive tokens at one chunk; this
// swizzle puts them on the 16 distinct 16-byte bank groups of a line.
//
// Score operand: 16-byte reads. Lane l holds token perm(l % 32) (bits 2 and 3
// swapped, so that the accumulator rows a lane owns are eight consecutive
// tokens) and 16-byte granule 2 s + l / 32 of the row. bf16: one read is one
// MFMA k-slice (36 reads per tile). fp8: one read holds the k-slices of two
// MFMAs (18 reads per tile); the query is loaded in the matching feature order.
//
// P . latent operand: transposed reads (ds_read_b64_tr_b16 / _b8) of output
// block 4 md + w for wave w (latent columns 128 md + 32 w .. +31), token half
// kk: a per-lane, per-wave base (one per 4-token half of a bf16 read) plus an
// immediate in (md, kk). In output round md the four waves together own 128
// consecutive columns.
template <bool KV8>
struct H128Layout {
    using G = TileLayout<KV8>;
    static constexpr int kTile = G::kTile, kRowBytes = G::kRowBytes, kCPT = G::kCPT;
    static constexpr int kCG = G::kCG, kTPB = G::kTPB, kNTB = G::kNTB, kNB = G::kNB;
    static constexpr int kTileBytes = G::kTileBytes;
    static constexpr int kTPL = 256 / (kCG * 16);  // tokens per 256-byte line: 2 | 4

    // Chunk swizzle of 256-byte line L = (t / kTPL) % kCG: a bijection (16
    // tokens of a score read reach 16 distinct 16-byte bank groups) that sends
    // lines 2m and 2m+1 to opposite halves of the chunk range (the 4 tokens of
    // a transposed P . latent read, two lines, reach distinct banks).
    static MLA_HD constexpr int swz(int t) {
        const int l = (t / kTPL) % kCG;
        return (l & 1) * (kCG / 2) + (l >> 1);
    }
    static MLA_HD constexpr int chunk_offset(int t, int j) {
        return ((j / kCG) * kNTB + t / kTPB) * 1024 + ((t % kTPB) * kCG + ((j % kCG) ^ swz(t))) * 16;
    }
    // Direct load of block (chunk group cg, token block tb): lane -> (token, chunk).
    static MLA_HD constexpr int block_token(int tb, int lane) { return tb * kTPB + lane / kCG; }
    static MLA_HD constexpr int block_chunk(int cg, int tb, int lane) {
        return cg * kCG + ((lane % kCG) ^ swz(block_token(tb, lane)));
    }

    static constexpr int kScoreReads = KV8 ? 18 : 36;
    static constexpr int kScoreBases = kCG / 2;
    static MLA_HD constexpr int score_token(int lane) {
        const int m = lane & 31;
        return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
    }
    static MLA_HD constexpr int score_ref(int lane, int s) {
        return chunk_offset(score_token(lane), 2 * s + (lane >> 5));
    }
    static MLA_HD constexpr int score_base_index(int s) { return s % kScoreBases; }
    static MLA_HD constexpr int score_delta(int s) { return score_ref(0, s) - score_ref(0, score_base_index(s)); }
    // First of the 8 features lane group g supplies to MFMA k-slice u (u < 36).
    static MLA_HD constexpr int q_feature(int u, int g) {
        return KV8 ? 32 * (u / 2) + 16 * g + 8 * (u % 2) : 16 * u + 8 * g;
    }

    static constexpr int kPvBases = KV8 ? 1 : 2;
    // Byte offset lane `lane` reads for output block blk (32 latent columns),
    // token half kk, 4-token half hi (bf16 only).
    static MLA_HD constexpr int pv_ref(int lane, int blk, int kk, int hi) {
        const int grp = lane >> 4, q = lane & 15;
        const int rowb = 16 * kk + 8 * (grp >> 1);
        const int colb = 32 * blk + 16 * (grp & 1);
        const int t = KV8 ? rowb + (q >> 1) : rowb + (q >> 2) + 4 * hi;
        const int cbyte = KV8 ? colb + 8 * (q & 1) : 2 * (colb + 4 * (q & 3));
        return chunk_offset(t, cbyte >> 4) + (cbyte & 15);
    }
    static MLA_HD constexpr int pv_base(int lane, int w, int hi) { return pv_ref(lane, w, 0, hi); }
    static MLA_HD constexpr int pv_delta(int md, int kk) { return pv_ref(0, 4 * md, kk, 0) - pv_ref(0, 0, 0, 0); }
    // Latent column of accumulator value r of output block 4 md + w, lane group g.
    static MLA_HD constexpr int column(int w, int md, int g, int r) {
        return 128 * md + 32 * w + 8 * (r / 4) + 4 * g + r % 4;
    }
};

// Output staging of the H=128 kernel: one round of [128 heads][128 columns]
// fp32, rows padded to 528 bytes so that 16 consecutive heads at the same
// column land on 16 distinct 4-bank groups.
struct OutStage {
    static constexpr int kRow = 528;
    static constexpr int kBytes = 128 * kRow;
    static MLA_HD int offset(int h, int col) { return h * kRow + 4 * col; }
};

// bf16 output staging of the H=128 kernel: [128 heads][512 / kRounds
// columns] per round, rows padded by 16 bytes (16-byte aligned; the 8-byte
// writes of the 32 heads of one write pass meet at most two to a bank group).
template <int kRounds>
struct OutStageBf16 {
    static constexpr int kCols = 512 / kRounds;
    static constexpr int kRow = 2 * kCols + 16;
    static constexpr int kBytes = 128 * kRow;
    static MLA_HD int offset(int h, int col) { return h * kRow + 2 * col; }
};

// Probabilities shared between the waves of the H=128 kernel: bf16
// [128 heads][32 tokens], rows padded to 80 bytes so that the 16-byte accesses
// of 16 consecutive heads fall on distinct LDS banks.
struct PBuf {
    static constexpr int kRow = 80;
    static constexpr int kBytes = 128 * kRow;
    // 8 consecutive tokens (16 bytes) starting at token 16 kk + 8 g of head h.
    static MLA_HD int offset(int h, int kk, int g) { return h * kRow + (16 * kk + 8 * g) * 2; }
};

// Pipeline depth (tile buffers in LDS) of a decode kernel instantiation.
// Bounded by 160 KiB of LDS per CU and by vmcnt (6 bits): the loads of
// stages-1 tiles must be countable.
template <int HW, int HS, bool KV8, bool OUT32>
struct Stages {
    static constexpr int kLoads = (TileLayout<KV8>::kNB + HS - 1) / HS;
    static constexpr int kByLds = (144 * 1024) / TileLayout<KV8>::kTileBytes;
    static constexpr int kByCnt = 1 + 63 / kLoads;
    // Four or more stages of the 32-heads-per-wave variant push its register
    // allocation (query + accumulators fill the file) into spilling.
    static constexpr int kCap = HW == 32 ? ((KV8 || OUT32) ? 2 : 3) : 6;
    static constexpr int value = kByLds < kByCnt ? (kByLds < kCap ? kByLds : kCap)
                                                 : (kByCnt < kCap ? kByCnt : kCap);
};

}  // namespace mla
