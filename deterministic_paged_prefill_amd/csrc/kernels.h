// Host-side launchers of the device kernels (defined in prefill.hip and merge.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "dpp_internal.h"

namespace dpp {

// Prefill items of one pass: num_items * num_kv_heads blocks of 64 * waves_for(head_dim)
// threads, dynamic LDS for the tile buffers and the item's page-id table. `narrow` selects the
// instantiation for tiles of at most kNarrowRows rows; block_n is the plan's KV tile
// (block_n_for(head_dim), or 32 for narrow bf16 tiles of an adaptive-tile comparison plan).
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int kv_dtype, bool narrow, int block_n,
                          hipStream_t stream);

// Merge of the split partials of one pass: grid (num_merges, num_kv_heads).
// max_tile_rows: the most rows a merged tile of the pass can have (a pass of narrow tiles has
// at most kNarrowRows); it sizes how many workgroups share a tile's rows.
hipError_t launch_merge(const MergeArgs& a, int head_dim, int num_kv_heads, int max_tile_rows, hipStream_t stream);

// Standalone merge over dense [rows, splits, heads, D] partials.
hipError_t launch_merge_dense(const MergeDenseArgs& a, hipStream_t stream);

}  // namespace dpp
