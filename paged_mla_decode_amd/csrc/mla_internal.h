// Internal declarations shared by the C-ABI layer, the host planner and the
// gfx950 kernels. Not part of the public interface.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

namespace mla {

constexpr int kLatent = 512;           // kv_lora_rank: the value width
constexpr int kRope = 64;              // qk_rope_head_dim
constexpr int kRow = kLatent + kRope;  // values per cached token
constexpr int kTile = 32;              // tokens per LDS tile in the decode kernel

// One decode kernel instantiation: HW heads per wave (MFMA N width), HS waves
// (head blocks) per workgroup, and how many such workgroups fit on one CU.
struct Variant {
    int hw;
    int hs;
    int wgs_per_cu;
    int item_cost;  // fixed cost of one work item, in 32-token tiles (measured)
    int rows_per_item = 1;  // MLA_DECODE_SHARED_ROWS: query rows of a request per item
};

// Selects the kernel instantiation for these parameters. Returns false when the
// parameters are outside what the library implements.
bool select_variant(const mla_decode_params* p, Variant* v);
const char* variant_name(const mla_decode_params* p);

// mla_decode_noalloc: the library's static device scratch (plan copy,
// partials, quantised query), 64 MiB per GPU, and its address on the current
// device (mla_noalloc.hip).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
int32_t noalloc_scratch(void** ptr);

// Host planner (pure host code, no HIP calls).
int32_t plan_bounds(const mla_decode_params* p, int32_t num_cus, int32_t batch, int32_t num_rows,
                    size_t* plan_bytes, size_t* workspace_bytes);
int32_t plan_build(const mla_decode_params* p, int32_t num_cus, int32_t batch,
                   const int32_t* qo_indptr, const int32_t* kv_indptr,
                   const int32_t* kv_last_page_len, void* plan_h, size_t plan_h_bytes);

struct DecodeArgs {
    const mla_work_item* items;
    const int32_t* workers;  // worker w processes items [workers[w], workers[w+1])
    const uint16_t* q_nope;  // bf16 bits
    int64_t qn_sn, qn_sh;
    const uint16_t* q_rope;
    int64_t qr_sn, qr_sh;
    const uint8_t* cache;
    const int32_t* kv_indices;
    const int32_t* kv_lens;  // may be null
    void* out;
    float* lse;  // may be null
    void* part_out;  // [partials][H][512]: bf16, or fp32 in the fp32-output mode
    float* part_lse;
    int32_t num_heads;
    int32_t page_size;
    int32_t page_shift;  // log2(page_size) when it is a power of two, else -1
    float scale_log2;    // sm_scale * kv_scale * log2(e)
    float out_scale;   // kv_scale (fp8 cache) or 1
    // 1: the bf16 tile loads carry the non-temporal hint (every request has one
    // query row, so each tile is read once per launch).
    int32_t stream_tiles;
    // Fused append (null c_new: none). The item flagged MLA_ITEM_LAST_CHUNK writes
    // its request's row L-1 from c_new/k_pe_new (bf16, row it.row) into cache_w
    // (the same memory as cache) before any of its tile loads.
    const uint16_t* c_new;
    int64_t c_new_sn;
    const uint16_t* k_pe_new;
    int64_t k_pe_new_sn;
    uint8_t* cache_w;
    float kv_scale;  // fp8 encoding divides by it
    // Fused prefix merge (null prefix_lse: none): the result is merged by LSE
    // with the state (prefix_out [N][H][512] in the output's precision,
    // prefix_lse [N][H]); unsplit rows in the decode kernel, split rows in the
    // merge kernels. out/lse may be the same memory as prefix_out/prefix_lse.
    const void* prefix_out;
    const float* prefix_lse;
    // Single-pass tree verify (null sfx_table: none). A row's last chunk (planned
    // sfx_max tokens longer than its request) takes tokens [L, L + sfx_lens[row])
    // from the pool rows sfx_table[row * sfx_stride + j] instead of the page table.
    const int32_t* sfx_table;
    int64_t sfx_stride;
    const int32_t* sfx_lens;
    int32_t sfx_max;
    // fp8 score (null q8: none): the query as e4m3fn codes, [rows][H][576]
    // (no-rope then rope features), and the exponent e of each row and head,
    // [rows][H]: query value = code * 2^e. The 128-head fp8 kernel only.
    const uint8_t* q8;
    const int32_t* q8_exp;
};

// Quantisation of the query for the fp8 score (one wave per query row and head).
// Rows at or past *dev_num_rows (the plan's device copy) are skipped, so that a
// graph-safe launch can cover max_rows rows.
struct QuantQueryArgs {
    const uint16_t* q_nope;
    int64_t qn_sn, qn_sh;
    const uint16_t* q_rope;
    int64_t qr_sn, qr_sh;
    int32_t num_heads;
    const int32_t* dev_num_rows;
    uint8_t* codes;
    int32_t* exps;
};
int launch_quantize_query(const QuantQueryArgs& q, int rows, void* stream);

// Decode kernel instantiations: the plain decode, the fused append, the fused
// prefix merge, the single-pass tree verify (128-head kernel only). The extra
// arguments of the last three never reach the first.
enum DecodeMode { kModePlain = 0, kModeAppend = 1, kModeMerge = 2, kModeTree = 3 };

// XCDs of an MI355X: workgroups go to them round robin.
constexpr int kXcds = 8;

// Single-pass tree verify: at most this many suffix slots per row.
constexpr int kMaxSuffixTokens = 256;

struct MergePartialsArgs {
    const mla_merge_item* merges;
    const void* part_out;  // as DecodeArgs::part_out
    const float* part_lse;
    void* out;
    float* lse;  // may be null
    int32_t num_heads;
    const void* prefix_out;  // fused prefix merge, or null
    const float* prefix_lse;
    // Graph-safe launches: the counts in the plan's device copy (null otherwise),
    // read by merge_partials_mixed_kernel.
    const int32_t* dev_num_merges;
    const int32_t* dev_num_wide;
    // merge_partials_mixed_kernel: its first wide_bound * H workgroups take the
    // wide merges; num_wide and num_merges are the counts when the device ones
    // are null (set by launch_merge_partials).
    int32_t wide_bound;
    int32_t num_wide;
    int32_t num_merges;
};

// Kernel launchers (device code lives in mla_kernels.hip). Return hipError_t as int.
int launch_decode(const Variant& v, int kv_dtype, int out_dtype, const DecodeArgs& a,
                  int num_workers, void* stream);
// The 128-head kernel (latent columns split across the waves), mla_decode_h128.hip.
int launch_decode_h128(int kv_dtype, int out_dtype, const DecodeArgs& a, int num_workers,
                       void* stream);
// Rows with at least kWideMergePartials partials are merged by a workgroup per
// row and head, the others by one wave per row and head (in the same launch
// when a plan has both kinds). The plan lists merges by partial count, most
// first; the first num_wide of them are wide.
constexpr int kWideMergePartials = 16;
int launch_merge_partials(int out_dtype, const MergePartialsArgs& a, int num_merges, int num_wide,
                          void* stream);
// Per-head product D[h][n][m] = sum_k A[h][m][k] B[h][n][k] in bf16 (fp32
// accumulation): element (h, m, k) of A at a[h*a_head + m*a_row + k], of B at
// b[h*b_head + n*b_row + k]; D at d[h*d_head + n*d_row + m]. Element strides.
struct HeadGemmArgs {
    const uint16_t* a;
    int64_t a_head, a_row;
    const uint16_t* b;
    int64_t b_head, b_row;
    void* d;
    int64_t d_head, d_row;
    int32_t n_rows;
};
// m_len a multiple of 128; k_len 128 or 512. mla_proj.hip.
int launch_head_gemm(const HeadGemmArgs& g, int num_heads, int m_len, int k_len, void* stream);
int launch_merge_states(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                        void* v_out, float* s_out, int64_t num_rows, int32_t head_dim,
                        int32_t v_dtype, void* stream);
int launch_tree_compact(const uint8_t* mask, int64_t mask_stride, const int32_t* req_to_token,
                        int64_t req_stride, const int32_t* prefix_lens, int32_t width,
                        int32_t num_rows, int32_t num_actual_rows, int32_t* page_table,
                        int64_t table_stride, int32_t* seqlens, void* stream);

}  // namespace mla
