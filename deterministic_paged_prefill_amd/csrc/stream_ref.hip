// Read-only streaming reference for the KV gather of a plan: every K and V byte the plan's
// prefill units read, each once, moved into LDS by LDS-DMA and discarded. No arithmetic, no
// barrier in the stream: it measures how fast this GPU can gather these pages with this grid,
// the ceiling the attention kernels' memory-bound launches (short extends, long decodes) are
// compared against.
//
// Grid: `split` workgroups of 512 threads per unit (item, kv head) of the plan, work index
// w = xcd_chunked(b, split * units) as in the attention launch, part = w % split. By keys:
// workgroup w covers the keys [lo + part * len / split, lo + (part + 1) * len / split) of its
// unit. By head_dim halves (split 2, DPP_STREAM_HEAD_SPLIT): workgroup w reads all of its
// unit's K and the part-th half of every V row, the gather of the head_dim-split attention
// launch. Each 64-lane load moves 1 KiB: 16-byte chunks of consecutive key rows (or half rows)
// of one tensor. A wave keeps DEPTH loads in flight (counted waits), into a ring of 16 one-KiB
// LDS slots per wave.
#include <hip/hip_runtime.h>

#include <string>

#include "kernels.h"
#include "plan.h"

namespace dpp {
namespace {

constexpr int kStreamThreads = 512;
constexpr int kSlots = 16;  // LDS slots of 1 KiB per wave
// page-id entries of one workgroup: a unit's keys lie in one 4096-token split, so its pages
// number at most 4096 / page_size + 2
constexpr int kTableEntries = kSplitTokens + 2;

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ inline void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds_base)
               : "memory");
}

struct StreamArgs {
  const int32_t* header;
  const unsigned char* k_pool;
  const unsigned char* v_pool;
  const int32_t* kv_indices;
  int64_t num_pages;
  int32_t item_offset;
  int32_t num_items;
  int32_t num_kv_heads;
  int32_t split;
  int32_t page_size;
  int32_t row_bytes;   // one key row of one kv head: head_dim x element size
  int32_t block_n;
  int32_t head_split;  // 1: split 2 by head_dim halves of V (all of K in both)
  uint32_t plan_id;
};

template <int DEPTH>
__global__ __launch_bounds__(kStreamThreads, 1) void stream_kernel(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const HeaderPreamble* pre = reinterpret_cast<const HeaderPreamble*>(a.header);
  if (pre->magic != kHeaderMagic || pre->plan_id != a.plan_id) return;
  const int units = a.num_items * a.num_kv_heads;
  const int w = xcd_chunked(blockIdx.x, a.split * units);
  const int part = w % a.split, u = w / a.split;
  const int kvh = u / a.num_items;
  const PrefillItem it = reinterpret_cast<const PrefillItem*>(a.header + a.item_offset)[u - kvh * a.num_items];
  const int key_lo = it.kv_tile_begin * a.block_n;
  const int key_hi = min(it.kv_tile_end * a.block_n, it.req.kv_len);
  const int len = max(key_hi - key_lo, 0);
  const int k0 = a.head_split ? key_lo : key_lo + (int)((int64_t)len * part / a.split);
  const int k1 = a.head_split ? key_lo + len : key_lo + (int)((int64_t)len * (part + 1) / a.split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks_per_row = a.row_bytes / 16;
  const int rows_per_load = 64 / chunks_per_row;
  // V: whole rows, or (head split) the part-th half of each row
  const int v_bytes = a.head_split ? a.row_bytes / 2 : a.row_bytes;
  const int v_chunks = v_bytes / 16;
  const int v_rows_per_load = 64 / v_chunks;
  const int64_t token_bytes = (int64_t)a.num_kv_heads * a.row_bytes;
  const int n_k = (k1 - k0 + rows_per_load - 1) / rows_per_load;
  const int n_v = (k1 - k0 + v_rows_per_load - 1) / v_rows_per_load;
  const int n_loads = n_k + n_v;  // K and V loads alternate while both remain
  const uint32_t ring = (uint32_t)(uintptr_t)smem + (uint32_t)wave * kSlots * 1024u;
  // this workgroup's page ids into LDS first: a page-id load inside the stream would make the
  // compiler wait for every DMA load in flight
  int32_t* table = reinterpret_cast<int32_t*>(smem + (kStreamThreads / 64) * kSlots * 1024);
  const int pg0 = k0 / a.page_size;
  const int n_pg = k1 > k0 ? (k1 - 1) / a.page_size - pg0 + 1 : 0;  // <= kTableEntries
  for (int j = threadIdx.x; j < n_pg; j += kStreamThreads) table[j] = a.kv_indices[it.req.page_start + pg0 + j];
  __syncthreads();
  int issued = 0;
  const int both = 2 * min(n_k, n_v);
  for (int i = wave; i < n_loads; i += kStreamThreads / 64) {
    const bool v = i < both ? (i & 1) : n_v > n_k;
    const int j = i < both ? i >> 1 : i - both + both / 2;  // index among this tensor's loads
    const int key = v ? k0 + j * v_rows_per_load + lane / v_chunks : k0 + j * rows_per_load + lane / chunks_per_row;
    const int col = v ? (a.head_split ? part * v_bytes : 0) + (lane % v_chunks) * 16 : (lane % chunks_per_row) * 16;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(pre->zero_chunk);
    if (key < k1) {
      const int pi = key / a.page_size;
      const int64_t pid = table[pi - pg0];
      if (pid >= 0 && pid < a.num_pages)
        src = (v ? a.v_pool : a.k_pool) + pid * (token_bytes * a.page_size) +
              (int64_t)(key - pi * a.page_size) * token_bytes + (int64_t)kvh * a.row_bytes + col;
    }
    if (issued >= DEPTH) wait_vm<DEPTH - 1>();
    dma16(src, __builtin_amdgcn_readfirstlane(ring + (uint32_t)(issued % kSlots) * 1024u));
    ++issued;
  }
  wait_vm<0>();  // no load may outlive the workgroup
}

template <int DEPTH>
hipError_t launch_stream(const StreamArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)(kStreamThreads / 64) * kSlots * 1024 + (size_t)kTableEntries * 4;
  static bool opted = false;
  if (!opted) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&stream_kernel<DEPTH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    opted = true;
  }
  hipLaunchKernelGGL(stream_kernel<DEPTH>, dim3((unsigned)(a.split * a.num_items * a.num_kv_heads)),
                     dim3(kStreamThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace dpp

using namespace dpp;

extern "C" dpp_status dpp_stream_kv(const dpp_plan* plan, const void* k_pool, const void* v_pool, int64_t num_pages,
                                    const int32_t* kv_indices, int64_t num_kv_indices, void* workspace,
                                    size_t workspace_bytes, int32_t split, int32_t depth, uint32_t flags,
                                    void* stream_ptr) {
  if (!plan) return fail(DPP_ERR_INVALID, "dpp_stream_kv: null plan");
  if (plan->ragged) return fail(DPP_ERR_UNSUPPORTED, "dpp_stream_kv: paged plans only");
  if (split < 1 || split > 8) return fail(DPP_ERR_INVALID, "dpp_stream_kv: split must be in [1, 8]");
  const bool head_split = (flags & DPP_STREAM_HEAD_SPLIT) != 0;
  if (head_split && split != 2) return fail(DPP_ERR_INVALID, "dpp_stream_kv: DPP_STREAM_HEAD_SPLIT needs split 2");
  if (depth != 4 && depth != 8 && depth != 16 && depth != 32)
    return fail(DPP_ERR_INVALID, "dpp_stream_kv: depth must be 4, 8, 16 or 32");
  if (num_pages < 0 || plan->total_kv_entries > num_kv_indices)
    return fail(DPP_ERR_SHAPE, "dpp_stream_kv: kv_indices shorter than kv_indptr[-1]");
  if (!k_pool || !v_pool || !kv_indices || !workspace) return fail(DPP_ERR_INVALID, "dpp_stream_kv: null pointer");
  if (workspace_bytes < plan->workspace_bytes || ((uintptr_t)workspace % 256) != 0)
    return fail(DPP_ERR_WORKSPACE, "dpp_stream_kv: workspace too small or misaligned");
  const int row_bytes = plan->cfg.head_dim * (plan->cfg.kv_dtype == DPP_KV_FP8_E4M3 ? 1 : 2);
  if (row_bytes % 16 != 0 || 64 % (row_bytes / 16) != 0)
    return fail(DPP_ERR_UNSUPPORTED, "dpp_stream_kv: key rows must split 1 KiB loads evenly");
  if (head_split && (row_bytes % 32 != 0 || 64 % (row_bytes / 32) != 0))
    return fail(DPP_ERR_UNSUPPORTED, "dpp_stream_kv: half rows must split 1 KiB loads evenly");
  if (flags & ~(DPP_RUN_REUSE_UPLOAD | DPP_STREAM_HEAD_SPLIT))
    return fail(DPP_ERR_INVALID, "dpp_stream_kv: unknown flags");
  if (plan->num_items == 0) return DPP_OK;
  if (!(flags & DPP_RUN_REUSE_UPLOAD)) {
    // the plan's work list must be in the workspace (upload it here, on this stream)
    const size_t hbytes = plan->header.size() * sizeof(int32_t);
    hipError_t e = hipMemcpyAsync(workspace, plan->header.data(), hbytes, hipMemcpyHostToDevice,
                                  (hipStream_t)stream_ptr);
    if (e != hipSuccess) return fail(DPP_ERR_HIP, std::string("dpp_stream_kv upload: ") + hipGetErrorString(e));
  }
  StreamArgs a{};
  a.header = (const int32_t*)workspace;
  a.k_pool = (const unsigned char*)k_pool;
  a.v_pool = (const unsigned char*)v_pool;
  a.kv_indices = kv_indices;
  a.num_pages = num_pages;
  a.item_offset = plan->item_offset;
  a.num_items = plan->num_items;
  a.num_kv_heads = plan->cfg.num_kv_heads;
  a.split = split;
  a.page_size = plan->cfg.page_size;
  a.row_bytes = row_bytes;
  a.block_n = plan->block_n;
  a.head_split = head_split ? 1 : 0;
  a.plan_id = plan->plan_id;
  hipError_t e;
  switch (depth) {
    case 4: e = launch_stream<4>(a, (hipStream_t)stream_ptr); break;
    case 8: e = launch_stream<8>(a, (hipStream_t)stream_ptr); break;
    case 16: e = launch_stream<16>(a, (hipStream_t)stream_ptr); break;
    default: e = launch_stream<32>(a, (hipStream_t)stream_ptr); break;
  }
  if (e != hipSuccess) return fail(DPP_ERR_HIP, std::string("dpp_stream_kv launch: ") + hipGetErrorString(e));
  return DPP_OK;
}
