// Internal definitions shared by the host planner (fia_plan.cpp) and the
// gfx950 kernels (fia_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "fia.h"

namespace fia {

enum Kind : int32_t { KIND_EMPTY = 0, KIND_PREFILL = 1, KIND_DECODE = 2, KIND_BSA = 3 };
enum Layout : int32_t { LAYOUT_BNSD = 0, LAYOUT_BSND = 1, LAYOUT_TND = 2 };

// Waves of a prefill workgroup (each 32 query rows of one head), query rows
// per block-sparse workgroup (4 waves), and kv tokens per inner step.
constexpr int kDenseWaves = 4;
constexpr int kBlockMSparse = 128;
constexpr int kBlockN = 64;
// XCDs of one MI355X: workgroup i of a launch runs on XCD i % kNumXcds.
constexpr int kNumXcds = 8;
// Tokens per inner step of the decode kernel; a decode split is a multiple.
constexpr int kDecodeStep = 32;
// Query rows (head, token) one decode wave serves; the G x S rows of a kv
// head are cut into chunks of this.
constexpr int kDecodeHeads = 16;
// Compute units of one MI355X and decode waves resident per CU, used only to
// size the decode schedule.
constexpr int kNumCUs = 256;
constexpr int kDecodeWavesPerCU = 8;
// Largest MLA decode workgroup (waves of 16 query rows each).
constexpr int kMlaMaxWaves = 8;
// Size of the static device scratch the allocation-free run uses as its
// workspace (FIA_NOALLOC_MAX_WORKSPACE in fia.h).
constexpr uint64_t kNoAllocScratchBytes = (uint64_t)32 << 20;

// Per-batch addressing, 24 bytes.  row0 is the first row of batch b on the
// tensor's row axis: b * S for BNSD/BSND, the cumulative start for TND.
struct BatchInfo {
    int64_t q_row0;
    int64_t kv_row0;
    int32_t lq;
    int32_t lkv;
};

// One prefill / block-sparse workgroup: query rows [q0, q1) of head h of
// batch b.  Rows at or past the batch's length (padding of BNSD/BSND) are
// written as out = 0, lse = +inf; rows at or past q1 are not touched.  The
// batch's addressing rides along (a copy of its BatchInfo), so a workgroup
// starts with one table load instead of two dependent ones.  40 bytes.
struct Tile {
    int32_t b, h, q0, q1;
    BatchInfo bi;
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const uint8_t* mask;           // explicit mask (modes 0/1), nonzero = masked
    int64_t mask_bstride;          // elements between batches (0 = broadcast)
    int64_t mask_rstride;          // elements between rows
    const Tile* tiles;             // workspace
    const BatchInfo* batch;        // workspace
    const int32_t* bsa_cnt;        // block-sparse schedule (workspace)
    const int32_t* bsa_idx;
    int32_t nqb, nkb, bx, by;      // block-sparse block counts and shape
    // element strides: head axis (sH) and sequence axis (sS)
    int64_t q_sH, q_sS, k_sH, k_sS, v_sH, v_sS, o_sH, o_sS, lse_sH, lse_sS;
    // row0 multipliers: base offset of batch b = row0 * mult
    int64_t q_rowmul, k_rowmul, v_rowmul, o_rowmul, lse_rowmul;
    int32_t QN, KVN, G;
    float scale_log2;              // scale_value * log2(e)
    int32_t mode;                  // sparse_mode 0..4
    int32_t has_mask;
    int64_t pre, next;
    int32_t return_lse;
    int32_t n_tiles;
    int32_t hg;                    // heads per dense workgroup (a divisor of G)
    // paged K/V (prefill): kv token j of batch b is row j % block_size of
    // pool block block_table[b][j / block_size]; k/v_sH and k/v_sS are then
    // the pool's head and token strides and p_blk its block stride
    const int32_t* block_table;
    int64_t bt_stride;
    int64_t p_blk;
    int32_t block_size;            // a multiple of 64 (tiles never cross a block)
    int32_t paged;
    // block-sparse FP8 (E4M3FN) inputs: fp32 dequant scales per (batch, head,
    // q block) and per (batch, kv head, kv block)
    int32_t fp8;
    const float* q_scale;          // [B, QN, nqb]
    const float* k_scale;          // [B, KVN, nkb]
    const float* v_scale;          // [B, KVN, nkb]
};

// Decode schedule.  The query rows of one (batch, kv head) are the G x S
// pairs (head of the GQA group, query token), row r = head * S + token; a
// segment is (batch b, kv head, chunk of <= 16 such rows) over kv tokens
// [0, Lkv_b).  The token streams of all segments are concatenated and cut
// into equal per-wave quotas; a piece is the part of one segment that one
// wave processes.
struct DecSeg {
    int64_t kv_row0;     // contiguous KV: first row of batch b
    int32_t b;
    int32_t lkv;
    int32_t first;       // first piece of this segment
    int32_t count;       // pieces of this segment (0 when lkv == 0)
    int32_t lq;          // valid query tokens of batch b (rows past it: out 0, lse +inf)
    int32_t q_row0;      // TND: first query row of batch b (else 0)
};

struct DecPiece {
    int32_t seg;         // (b * KV_N + kv head) * nhc + head chunk
    int32_t t0, t1;      // kv tokens [t0, t1), t0 % 16 == 0
    int32_t pad;
};

struct DecodeArgs {
    const void* q;                 // [B, QN, S, D] / [B, S, QN, D] / [B, S, QN*D]
    const void* k;
    const void* v;
    void* o;                       // the query's layout with D = Dv
    float* lse;                    // [B, QN, S, 1]
    // query / output element strides: batch, head, token
    int64_t q_sB, q_sH, q_sS, o_sB, o_sH, o_sS;
    int32_t S;                     // query tokens per sequence (<= 16)
    int32_t causal;                // sparse_mode 3: token t sees keys j <= Lkv - Lq + t
    // query S == 1 atten_mask, one byte per (batch, kv token), nonzero =
    // masked; batch b's row starts at mask + b * mask_bstride (0: broadcast)
    const uint8_t* mask;
    int64_t mask_bstride;
    // int8 key/value (kv pseudo-quantization): dequantized value
    // scale * (x + offset); mode 0 per channel (bf16 [KV_N * D]), mode 1 per
    // token (fp32 [B, tok_stride]); offsets nullable (0)
    int32_t kv_i8;
    int32_t kmode, vmode;
    const void* k_scale;
    const void* k_off;
    const void* v_scale;
    const void* v_off;
    int64_t tok_stride;
    const int32_t* block_table;    // paged only
    int64_t bt_stride;
    int32_t block_size;            // paged only
    int32_t paged;
    // paged pool strides (elements): block, kv head, token
    int64_t p_blk, p_head, p_tok;
    // contiguous strides (elements): head, token, and row0 multiplier
    int64_t c_head, c_tok, c_rowmul;
    const DecSeg* segs;            // plan tables
    const DecPiece* pieces;
    const int32_t* wave_first;     // [n_waves + 1]: pieces of wave w
    float* part_o;                 // [n_pieces, Gc, Dv]
    float* part_lse;               // [n_pieces, Gc]
    int32_t B, QN, KVN, G, Gc, nhc; // Gc rows per chunk, nhc chunks of G * S rows
    int32_t n_waves, n_pieces;
    float scale_log2;
    int32_t return_lse;
    // MLA: query_rope (the query's layout, D 64; element strides batch, head,
    // token), the key_rope pool (block stride pr_blk, token stride 64) and
    // the waves per workgroup (0 = not MLA)
    const void* qr;
    const void* kr;
    int64_t qr_sB, qr_sH, qr_sS;
    int64_t pr_blk;
    int32_t mla_nw;
    int32_t tnd;                   // TND query (MLA): rows q_row0 + t; rows t >= Lq do not exist
    // MLA: query token t sees keys Lkv - Lq + t + band_lo .. Lkv - Lq + t + band_hi
    int32_t band_lo, band_hi;
    int32_t v_is_k;                // value is the key tensor itself (V read from the K tile)
};

}  // namespace fia

struct fia_plan {
    int32_t kind = fia::KIND_EMPTY;
    int32_t dtype = FIA_BF16;
    int32_t layout = fia::LAYOUT_BNSD;
    int64_t B = 0, QN = 0, KVN = 0, G = 0, Sq = 0, Skv = 0, Dqk = 0, Dv = 0;

    // Schedule tables: built on the host, uploaded once by phase 1 into a
    // device buffer the plan owns (dev_tables).
    void* dev_tables = nullptr;
    uint64_t tables_bytes = 0;
    uint64_t workspace_bytes = 0;

    // byte offsets inside dev_tables
    uint64_t off_batch = 0, off_tiles = 0, off_pieces = 0, off_waves = 0;
    // byte offsets inside the caller's workspace
    uint64_t off_part_o = 0, off_part_lse = 0;
    uint64_t off_cnt = 0, off_idx = 0;

    int64_t n_tiles = 0;     // prefill / block-sparse workgroups
    int64_t n_waves = 0;     // decode waves
    int64_t n_pieces = 0;    // decode pieces (partial results)
    int64_t n_rows = 0;      // block-sparse compaction rows (B * N1 * nqb)

    fia::AttnArgs attn{};
    fia::DecodeArgs dec{};
    const uint8_t* bsa_mask = nullptr;
    int64_t bsa_nqb = 0, bsa_nkb = 0;
};

namespace fia {
// Kernel launchers (fia_kernels.hip).  Return 0 on success, else a HIP error.
int launch_prefill(const fia_plan& p, const AttnArgs& a, void* stream);
int launch_decode(const fia_plan& p, const DecodeArgs& a, void* stream);
int launch_bsa(const fia_plan& p, const AttnArgs& a, void* stream);
// Device copy of a plan's schedule tables (synchronous); nullptr on failure.
void* upload_tables(const void* src, uint64_t bytes);
// Device address of the current device's static scratch array (resolved
// once per device); nullptr when no device is current or the lookup fails.
void* noalloc_scratch();
void free_tables(void* dev);
}  // namespace fia
