// Internal constants and work-list record formats of libdpp (not part of the C ABI).
//
// Fixed arithmetic constants. Together with the MFMA instruction shapes and the softmax code
// in prefill.hip, these decide every bit of a row. They depend on nothing about the batch;
// this is how a prefix-cache hit reproduces the full prefill (the sglang PR #46351 page,
// "Root cause", shows FlashInfer losing that property by sizing its q tile from the batch's
// average query length).
#pragma once

#include <cstddef>
#include <cstdint>

#if defined(__HIPCC__)
#define DPP_HOST_DEVICE __host__ __device__
#else
#define DPP_HOST_DEVICE
#endif

namespace dpp {

// Tile geometry: constants of head_dim, never of the batch.
// A packed query row is (token, q head within the kv head's group); row R of a request covers
// token R / group and q head kv_head * group + R % group. A wave owns 32 packed rows as two
// 16-row MFMA column blocks at head_dim <= 128 and one 16-row block at 256 and 512 (where a
// row's fp32 output takes 64 and 128 registers of a wave's lanes); a workgroup is 8 waves (two
// per SIMD: 256-row tiles at head_dim <= 128, 128-row tiles at 256) or 4 waves (one per SIMD,
// 64-row tiles) at 512.
DPP_HOST_DEVICE constexpr int rows_per_wave_for(int head_dim) { return head_dim <= 128 ? 32 : 16; }
DPP_HOST_DEVICE constexpr int waves_for(int head_dim) { return head_dim <= 256 ? 8 : 4; }
DPP_HOST_DEVICE constexpr int block_m_for(int head_dim) {
  return rows_per_wave_for(head_dim) * waves_for(head_dim);
}
// A q tile with at most this many rows (a short extend) is run by a narrow instantiation of
// the same kernel whose waves hold one 16-row block. Which instantiation runs a tile is a
// launch choice: the per-row arithmetic is the same.
constexpr int kNarrowRows = 16;
// Keys per KV tile. Tiles start at absolute key positions 0, BN, 2BN, ...
DPP_HOST_DEVICE constexpr int block_n_for(int head_dim) { return head_dim <= 128 ? 64 : 32; }
constexpr int kMaxBlockM = 256;
// Largest group (q heads per kv head): the kernels split a packed row into (token, q head)
// with a multiply-shift that is exact for groups up to this size.
constexpr int kMaxGroup = 1024;
// LDS of a workgroup: a ring of K and V tiles (bf16) -- four of each, two at head_dim 512
// whose 32-key tiles are 32 KiB -- then page-id tables (4 bytes an entry; two in a persistent
// launch, one per unit in flight), within the 160 KiB of a CU.
DPP_HOST_DEVICE constexpr int ring_buffers_for(int head_dim) { return head_dim <= 256 ? 4 : 2; }
DPP_HOST_DEVICE constexpr int ring_bytes_for(int head_dim) {
  return 2 * ring_buffers_for(head_dim) * block_n_for(head_dim) * head_dim * 2;
}
constexpr int kLdsLimit = 160 * 1024;
// Output staging of the two-group schedule: 2 KiB for each wave of a group.
constexpr int kOutStageBytes = 4 * 2048;
// Bytes of one page-id table for units spanning up to page_slots pages: the ids arrive by
// whole 64-entry DMA loads, and the last KV tile may look up to one tile of keys past kv_len.
DPP_HOST_DEVICE constexpr int64_t page_table_bytes(int64_t page_slots, int head_dim) {
  return ((page_slots + 63) / 64 * 64 + block_n_for(head_dim)) * 4;
}
constexpr int kMergeThreads = 256;

// Fixed KV split length (the model-serving-minefield issue #73 correction comment,
// "What the flag actually does", item 2). Splits start at absolute positions 0, 4096, ...
// Blocks of a launch are dispatched round-robin over the chip's XCDs (8 on MI355X, each with
// its own L2). xcd_chunked maps block b of n to a work index so that XCD x receives the
// contiguous range [x*q + min(x, r), +q + (x < r)), q = n / kXcds, r = n % kXcds, in order.
// It is a bijection on [0, n) for any kXcds; only locality depends on the value.
constexpr int kXcds = 8;
DPP_HOST_DEVICE inline int xcd_chunked(int b, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int x = b % kXcds;
  return x * q + (x < r ? x : r) + b / kXcds;
}

// Persistent launches. A wide bf16 launch at head_dim <= 256 (eight waves) runs as this many
// workgroups -- one per compute unit of an MI355X; the LDS ring leaves room for one workgroup
// per CU -- each working through a chain of units (item, kv head) fixed by the planner. The
// chain a unit lands in decides when it runs, never its arithmetic.
constexpr int kPersistentBlocks = 256;
// Planner's cost estimate of a unit: its KV tiles plus this many tiles' worth of start-up.
constexpr int kUnitOverheadTiles = 2;
DPP_HOST_DEVICE constexpr bool chained_launch(int head_dim, bool fp8, bool narrow) {
  return !fp8 && !narrow && waves_for(head_dim) == 8;
}

constexpr int kSplitTokens = 4096;
// Ragged (contiguous) KV: one virtual page per request, this many tokens long, whose id is 0
// (read from the work list's zero chunk) and whose base is the request's first token.
constexpr int kRaggedPage = 1 << 30;
static_assert(kSplitTokens % 64 == 0 && kSplitTokens % 32 == 0, "splits must be whole KV tiles");

constexpr uint32_t kHeaderMagic = 0x44505031u;  // "DPP1"
constexpr int kHeaderWords = 16;                // fixed preamble (see HeaderPreamble)

// ---- work-list records (int32 words, uploaded to the head of the workspace) ----

// Per request: where its query rows start in q, how many, where its page list starts in
// kv_indices, and how many KV tokens it has.
struct RequestDesc {
  int32_t q_start;
  int32_t qo_len;
  int32_t page_start;
  int32_t kv_len;
};

// One (q tile, KV split) unit of the prefill kernel, run once per kv head. It carries a copy
// of its request's descriptor, so a workgroup reads one record before it can start loading.
struct PrefillItem {
  int32_t request;
  int32_t row_start;     // first packed row of the tile (multiple of block_m_for(head_dim))
  int32_t split;         // split index s; keys [s*4096, (s+1)*4096)
  int32_t tile_splits;   // splits the tile's last row needs (S_t)
  int32_t kv_tile_begin; // first KV tile (absolute, units of block_n_for(head_dim))
  int32_t kv_tile_end;   // one past the last KV tile this item visits
  int32_t slot_base;     // first partial slot of the tile in this pass, -1 if S_t == 1
  int32_t pass;          // the pass (launch group) that runs the item; the kernels ignore it
  RequestDesc req;       // the request's descriptor
  int32_t pad1[4];
};
// Unit record of a persistent launch: the item's record with four words reused. Workgroup b
// of the launch starts at record b of its pass and follows `next` (an index into the pass's
// records, -1 after its last unit).
struct UnitRecord {
  int32_t request, row_start, split, tile_splits, kv_tile_begin, kv_tile_end, slot_base;
  int32_t next;
  RequestDesc req;
  int32_t kv_head;
  int32_t block;         // workgroup that runs it
  int32_t pass;
  int32_t pad;
};
static_assert(sizeof(UnitRecord) == sizeof(PrefillItem), "unit record is an item record");
static_assert(sizeof(PrefillItem) == 64, "item record is 16 words");
constexpr int kItemWords = 16;

// One q tile whose rows span several splits: merge its partials.
struct MergeItem {
  int32_t request;
  int32_t row_start;
  int32_t tile_splits;
  int32_t slot_base;
};

// Rows of a q tile's slot block per (kv head, split): the tile's rows rounded up to 16, so a
// short tile (an extend or a one-token decode) does not hold a full tile's worth of slots.
DPP_HOST_DEVICE constexpr int slot_rows_for(int tile_rows) { return (tile_rows + 15) / 16 * 16; }
// Partial slot of (kv head c, split s, tile-local row lr) inside a tile's slot block, with
// block_m = slot_rows_for(the tile's rows).
DPP_HOST_DEVICE inline int64_t partial_slot(int32_t slot_base, int32_t tile_splits, int c, int s,
                                            int lr, int block_m) {
  return (int64_t)slot_base + ((int64_t)c * tile_splits + s) * block_m + lr;
}

struct HeaderPreamble {
  uint32_t magic;
  int32_t num_requests;
  int32_t num_items;
  int32_t num_merges;
  int32_t request_offset;  // word offsets from the start of the header
  int32_t item_offset;
  int32_t merge_offset;
  uint32_t plan_id;        // unique per plan; kernels refuse a header with another id
  int32_t zero_chunk[4];   // zero: the gather reads these 16 bytes in place of a missing chunk
  int32_t unit_offset;     // word offset of the unit records (all passes), 0 if none
  int32_t num_units;
  int32_t table_offset;    // word offset of the block tables (pass, blocks, entries...), 0 if none
  int32_t num_tables;
};
static_assert(sizeof(HeaderPreamble) == kHeaderWords * 4, "preamble size");
static_assert(offsetof(HeaderPreamble, zero_chunk) % 16 == 0, "zero chunk must be 16-byte aligned");

// ---- kernel launch arguments ----

struct PrefillArgs {
  const void* q;            // bf16 [rows, Hq, D]
  const void* k_pool;       // [pages, page_size, Hkv, D] bf16 or e4m3
  const void* v_pool;
  const int32_t* kv_indices;
  void* o;                  // bf16 [rows, Hq, D]
  float* lse;               // [rows, Hq]
  const int32_t* header;    // device copy of the work list
  float* part_o;            // [slots, D]
  float* part_lse2;         // [slots] (base-2 log-sum-exp of the split)
  int64_t num_pages;
  uint32_t plan_id;
  int32_t item_offset;      // word offset of the item records in the header
  int32_t item_begin;       // first item of this launch
  int32_t num_items;        // items in this launch
  int32_t chain_offset;     // persistent launch: word offset of its unit records; -1: see
                            // block_table
  int32_t num_chains;       // persistent launch: its workgroups (one per chain)
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t page_size;        // kRaggedPage for a ragged (contiguous) KV layout
  int32_t page_slots;       // entries of one unit's page-id table in LDS
  int32_t ragged;           // 1: K/V are [tokens, Hkv, D]; a request's page_start is its first
                            // token and its keys sit on one virtual page with id 0
  int32_t block_table;      // wide launch that is not persistent: word offset of its block table
                            // (block b runs unit table[b], or exits at -1); -1: block b runs unit
                            // xcd_chunked(b, num_items * num_kv_heads)
  int32_t table_blocks;     // entries of that table: the launch's workgroups
  float scale_log2;         // sm_scale * log2(e), rounded once to fp32
  float k_scale;
  float v_scale;
  int32_t kv_scale_pow2;    // fp8: both scales are powers of two in [2^-64, 2^64]
  uint32_t pool_bytes;      // bytes of one pool (num_pages x page bytes) if below 2^32 - 64, else 0
};

struct MergeArgs {
  const int32_t* header;
  const float* part_o;
  const float* part_lse2;
  void* o;
  float* lse;
  uint32_t plan_id;
  int32_t merge_begin;
  int32_t num_merges;
  int32_t num_qo_heads;
  int32_t group;
  int32_t block_m;
};

// Standalone merge over [rows, splits, heads, D] partials with natural-log lse.
struct MergeDenseArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int64_t num_rows;
  int32_t num_splits;
  int32_t num_heads;
  int32_t head_dim;
};

}  // namespace dpp
