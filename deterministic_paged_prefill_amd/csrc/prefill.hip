// Causal GQA prefill attention over a paged KV cache, gfx950 (CDNA4), wave64.
//
// One workgroup = one (q tile of kBlockM packed rows, KV split, kv head). Four waves each own
// 32 packed rows. Per KV tile of kBlockN = 64 keys:
//   gather   K and V rows through the page table into LDS (K row-major, V transposed),
//            keys past kv_len zero-filled; fp8 E4M3 pages are decoded to bf16 on the way;
//   QK^T     S^T[key, row] = K Q^T on v_mfma_f32_32x32x16_bf16, fp32 accumulation over
//            head_dim in ascending 16-wide chunks (keys on M, this wave's 32 rows on N, so
//            every lane holds scores of a single query row);
//   mask     keys past the row's position p = kv_len - qo_len + token get -inf (a select
//            after identical arithmetic; tiles wholly below the diagonal skip the select,
//            which would not change a bit there);
//   softmax  online, fp32, base 2: m' = max(m, max_j s_j); alpha = 1 if m' == m else
//            exp2(m*c - m'*c); P_j = exp2(fma(s_j, c, -m'*c)); l = fma(l, alpha, sum_j P_j)
//            with the row sum taken in one fixed tree (c = sm_scale * log2 e);
//   PV       O^T[d, row] = alpha * O^T + V^T P^T on the same MFMA, P rounded to bf16 (RNE).
// After a split's last tile a row either writes o = O / l (bf16) and lse = (m*c + log2 l) ln 2,
// or -- when its keys reach past 4096 -- writes the split's fp32 partial (O / l, m*c + log2 l)
// for the merge kernel.
//
// Why this is batch invariant: a row's bits depend on its query, keys 0..p, the tile and split
// grid (absolute positions), the MFMA shapes and the code above. Which tile, wave or lane the
// row lands in, how many rows share its tile, and how many other requests run beside it do
// not enter its arithmetic: rows never mix inside an MFMA column, every lane runs the same
// reduction tree, and tiles past a row's position are exact no-ops for it (alpha = 1, P = 0,
// V zero-filled past kv_len). This replaces the fix the sglang PR #46351 page describes
// (front-padding q so FlashInfer keeps its q-tile size) with a design that has no
// batch-dependent choice to pin.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "dpp_internal.h"
#include "kernels.h"

namespace dpp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;

template <int D>
struct Geometry {
  static constexpr int kChunks = D / 8;                 // 16-byte bf16 chunks per K/V row
  static constexpr int kRowsPerPass = kThreads / kChunks;
  static constexpr int kPasses = kBlockN / kRowsPerPass;  // K rows each thread stages
  static constexpr int kGroupsPerPass = kThreads / kChunks;  // 4-key groups per V pass
  static constexpr int kVPasses = kBlockN / (4 * kGroupsPerPass);
  static constexpr int kStrideK = D + 8;       // bf16 elements per K row in LDS (16 B pad)
  static constexpr int kStrideV = kBlockN + 4;  // bf16 elements per V^T row in LDS (8 B pad)
  static constexpr int kBytesK = kBlockN * kStrideK * 2;
  static constexpr int kBytesV = D * kStrideV * 2;
  static constexpr int kDChunks = D / 16;  // MFMA k-steps over head_dim
  static constexpr int kDBlocks = D / 32;  // 32-row blocks of O^T
  static_assert(kPasses * kRowsPerPass == kBlockN, "K staging");
  static_assert(kVPasses * 4 * kGroupsPerPass == kBlockN, "V staging");
};

// OCP E4M3 code -> fp32 (exact): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
// S.1111.111 is NaN, no infinities.
__device__ inline float e4m3_to_f32(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t em = code & 0x7Fu;
  if (em == 0x7Fu) return __uint_as_float(0x7FC00000u | sign);
  if (em < 8u) {  // subnormal: m * 2^-9
    return __uint_as_float(sign | __float_as_uint((float)em * 0.001953125f));
  }
  return __uint_as_float(sign | ((em + (120u << 3)) << 20));
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// 8 E4M3 codes (two dwords) -> 8 bf16 (four dwords), value = decode(code) * scale.
__device__ inline u32x4 dequant8(u32x2 raw, float scale) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t x = raw[w];
    const float f0 = e4m3_to_f32(x & 0xFFu) * scale;
    const float f1 = e4m3_to_f32((x >> 8) & 0xFFu) * scale;
    const float f2 = e4m3_to_f32((x >> 16) & 0xFFu) * scale;
    const float f3 = e4m3_to_f32(x >> 24) * scale;
    out[2 * w] = pack_bf16x2(f0, f1);
    out[2 * w + 1] = pack_bf16x2(f2, f3);
  }
  return out;
}

// Raw storage of one staged 8-element chunk: 16 B (bf16) or 8 B (fp8).
template <bool FP8>
struct Chunk;
template <>
struct Chunk<false> {
  u32x4 v;
};
template <>
struct Chunk<true> {
  u32x2 v;
};

template <int D, bool FP8>
__device__ inline Chunk<FP8> load_chunk(const void* pool, int64_t elem) {
  Chunk<FP8> c;
  if constexpr (FP8) {
    c.v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(pool) + elem);
  } else {
    c.v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(pool) + elem);
  }
  return c;
}

template <bool FP8>
__device__ inline Chunk<FP8> zero_chunk() {
  Chunk<FP8> c;
  if constexpr (FP8) {
    c.v = u32x2{0u, 0u};
  } else {
    c.v = u32x4{0u, 0u, 0u, 0u};
  }
  return c;
}

template <bool FP8>
__device__ inline u32x4 to_bf16(const Chunk<FP8>& c, float scale) {
  if constexpr (FP8) {
    return dequant8(c.v, scale);
  } else {
    (void)scale;
    return c.v;
  }
}

// Element offset of (token j, kv head c, chunk ch) in a pool, or -1 when j is past kv_len or
// its page id is out of range (the chunk is then staged as zeros).
__device__ inline int64_t pool_offset(int j, int kv_len, int key_lo_page, int page_size,
                                      int page_shift, const int32_t* pg_lds, int64_t num_pages,
                                      int64_t token_stride, int64_t head_off) {
  if (j >= kv_len) return -1;
  int pi, slot;
  if (page_shift >= 0) {
    pi = j >> page_shift;
    slot = j & (page_size - 1);
  } else {
    pi = j / page_size;
    slot = j - pi * page_size;
  }
  const int64_t page = pg_lds[pi - key_lo_page];
  if (page < 0 || page >= num_pages) return -1;
  return (page * page_size + slot) * token_stride + head_off;
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  using G = Geometry<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* k_lds = reinterpret_cast<uint16_t*>(smem);
  uint16_t* vt_lds = reinterpret_cast<uint16_t*>(smem + G::kBytesK);
  int32_t* pg_lds = reinterpret_cast<int32_t*>(smem + G::kBytesK + G::kBytesV);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = blockIdx.y;

  const HeaderPreamble* pre = reinterpret_cast<const HeaderPreamble*>(a.header);
  if (pre->magic != kHeaderMagic || pre->plan_id != a.plan_id) return;  // not this plan's work list
  const PrefillItem it =
      reinterpret_cast<const PrefillItem*>(a.header + pre->item_offset)[a.item_begin + blockIdx.x];
  const RequestDesc rq = reinterpret_cast<const RequestDesc*>(a.header + pre->request_offset)[it.request];

  const int g = a.group;
  const int rows_total = rq.qo_len * g;
  const int tile_rows = min(kBlockM, rows_total - it.row_start);
  const int ctx = rq.kv_len - rq.qo_len;  // position of query token 0
  const int n = lane & 31;                  // this lane's query row within the wave
  const int hf = lane >> 5;                 // which half of the MFMA k-group the lane feeds
  const int lr = wave * 32 + n;             // tile-local packed row
  const int R = it.row_start + lr;
  const bool row_valid = lr < tile_rows;
  const int token = R / g;
  const int qhead = kvh * g + (R - token * g);
  // Rows past the tile are given a position no key reaches, so they stay finite (q = 0).
  const int p = row_valid ? ctx + token : INT_MAX;
  const int p_min = ctx + it.row_start / g;  // smallest position in the tile
  const int split_key0 = it.split * kSplitTokens;

  // ---- page ids of the keys this item visits -> LDS
  const int page_size = a.page_size;
  const int page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz(page_size) : -1;
  const int key_lo = it.kv_tile_begin * kBlockN;
  const int key_hi = min(it.kv_tile_end * kBlockN, rq.kv_len);
  const int key_lo_page = key_lo / page_size;
  const int n_pages = key_hi > key_lo ? (key_hi - 1) / page_size - key_lo_page + 1 : 0;
  for (int i = tid; i < n_pages; i += kThreads) pg_lds[i] = a.kv_indices[rq.page_start + key_lo_page + i];

  // ---- this lane's query row, as the MFMA B operand (16-byte chunks of head_dim)
  bf16x8 qreg[G::kDChunks];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((int64_t)(rq.q_start + token) * a.num_qo_heads + qhead) * D + hf * 8;
#pragma unroll
    for (int kc = 0; kc < G::kDChunks; ++kc) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row_valid) v = *reinterpret_cast<const u32x4*>(qrow + kc * 16);
      qreg[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();  // page table visible

  // ---- staging assignments
  const int64_t token_stride = (int64_t)a.num_kv_heads * D;
  const int64_t head_off = (int64_t)kvh * D;
  const int kch = tid % G::kChunks;     // chunk this thread stages
  const int krow0 = tid / G::kChunks;   // first K row
  const int vgrp0 = tid / G::kChunks;   // first 4-key V group
  Chunk<FP8> kst[G::kPasses];
  Chunk<FP8> vst[G::kVPasses][4];

  auto load_tile = [&](int kt) {
    const int base = kt * kBlockN;
#pragma unroll
    for (int i = 0; i < G::kPasses; ++i) {
      const int j = base + krow0 + i * G::kRowsPerPass;
      const int64_t off = pool_offset(j, rq.kv_len, key_lo_page, page_size, page_shift, pg_lds,
                                      a.num_pages, token_stride, head_off);
      kst[i] = off >= 0 ? load_chunk<D, FP8>(a.k_pool, off + kch * 8) : zero_chunk<FP8>();
    }
#pragma unroll
    for (int i = 0; i < G::kVPasses; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = base + 4 * (vgrp0 + i * G::kGroupsPerPass) + e;
        const int64_t off = pool_offset(j, rq.kv_len, key_lo_page, page_size, page_shift, pg_lds,
                                        a.num_pages, token_stride, head_off);
        vst[i][e] = off >= 0 ? load_chunk<D, FP8>(a.v_pool, off + kch * 8) : zero_chunk<FP8>();
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < G::kPasses; ++i) {
      const int r = krow0 + i * G::kRowsPerPass;
      *reinterpret_cast<u32x4*>(k_lds + r * G::kStrideK + kch * 8) = to_bf16<FP8>(kst[i], a.k_scale);
    }
#pragma unroll
    for (int i = 0; i < G::kVPasses; ++i) {
      const int k0 = 4 * (vgrp0 + i * G::kGroupsPerPass);
      u32x4 rows[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) rows[e] = to_bf16<FP8>(vst[i][e], a.v_scale);
      // transpose: element t of the chunk, keys k0..k0+3 -> V^T[kch*8 + t][k0 .. k0+3]
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int w = t >> 1;
        const int sh = (t & 1) * 16;
        const uint32_t x0 = (rows[0][w] >> sh) & 0xFFFFu;
        const uint32_t x1 = (rows[1][w] >> sh) & 0xFFFFu;
        const uint32_t x2 = (rows[2][w] >> sh) & 0xFFFFu;
        const uint32_t x3 = (rows[3][w] >> sh) & 0xFFFFu;
        *reinterpret_cast<u32x2*>(vt_lds + (kch * 8 + t) * G::kStrideV + k0) =
            u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
      }
    }
  };

  // ---- online-softmax state of this lane's row
  const float c = a.scale_log2;
  float m_raw = -INFINITY;  // running max of raw scores
  float m_sc = -INFINITY;   // m_raw * c
  float l = 0.f;
  f32x16 acc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  load_tile(it.kv_tile_begin);
  for (int kt = it.kv_tile_begin; kt < it.kv_tile_end; ++kt) {
    __syncthreads();  // everyone is done reading the previous tile
    store_tile();
    __syncthreads();  // tile kt visible
    if (kt + 1 < it.kv_tile_end) load_tile(kt + 1);

    // S^T = K Q^T for keys [kt*64, kt*64+64): two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 accs;
#pragma unroll
      for (int r = 0; r < 16; ++r) accs[r] = 0.f;
      const uint16_t* krow = k_lds + (kb * 32 + n) * G::kStrideK + hf * 8;
#pragma unroll
      for (int kc = 0; kc < G::kDChunks; ++kc) {
        const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + kc * 16));
        accs = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qreg[kc], accs, 0, 0, 0);
      }
      s[kb] = accs;
    }

    // causal mask: key index of s[kb][r] is kt*64 + kb*32 + (r/4)*8 + hf*4 + r%4
    const int key0 = kt * kBlockN;
    if (key0 + kBlockN - 1 > p_min) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
          s[kb][r] = key > p ? -INFINITY : s[kb][r];
        }
    }

    // row max: this lane's 32 scores, then the partner lane holding the row's other 32
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    const float m_new = fmaxf(m_raw, mx);
    const float m_new_sc = m_new * c;
    const float alpha = (m_new == m_raw) ? 1.f : __builtin_amdgcn_exp2f(m_sc - m_new_sc);
    m_raw = m_new;
    m_sc = m_new_sc;

    float pv[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_new_sc));

    // row sum: fixed pairwise tree over the lane's 32 values, then + partner's
    float t16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t16[i] = pv[i >> 3][(2 * i) & 15] + pv[i >> 3][(2 * i + 1) & 15];
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) t16[i] = t16[2 * i] + t16[2 * i + 1];
    const float rs = t16[0] + __shfl_xor(t16[0], 32);
    l = __builtin_fmaf(l, alpha, rs);

    if (__any(alpha != 1.f)) {  // acc * 1 == acc: skipping keeps every bit
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }

    // O^T += V^T P^T. MFMA (kb, u) covers keys kb*32 + 16u + [0, 16); its k index
    // 8*hf + t is key kb*32 + 16u + 8*(t/4) + 4*hf + t%4, i.e. the lane's P values
    // s[kb][8u .. 8u+7] and V^T rows read at those key offsets.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 pb;
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[w] = pack_bf16x2(pv[kb][8 * u + 2 * w], pv[kb][8 * u + 2 * w + 1]);
        const bf16x8 pbf = __builtin_bit_cast(bf16x8, pb);
        const int kofs = kb * 32 + 16 * u + 4 * hf;
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db) {
          const uint16_t* vrow = vt_lds + (db * 32 + n) * G::kStrideV + kofs;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbf, acc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: this lane holds O^T[d][row] for d = db*32 + (r/4)*8 + 4*hf + r%4
  if (!row_valid || p < split_key0) return;  // not a row of this split
  const float inv_l = 1.f / l;
  const float lse2 = m_sc + __builtin_amdgcn_logf(l);
  const int row_splits = p / kSplitTokens + 1;
  if (row_splits == 1) {
    const int64_t orow = (int64_t)(rq.q_start + token) * a.num_qo_heads + qhead;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + orow * D + 4 * hf;
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i;
        *reinterpret_cast<u32x2*>(op + db * 32 + i * 8) =
            u32x2{pack_bf16x2(acc[db][r] * inv_l, acc[db][r + 1] * inv_l),
                  pack_bf16x2(acc[db][r + 2] * inv_l, acc[db][r + 3] * inv_l)};
      }
    if (hf == 0) a.lse[orow] = lse2 * kLn2;
  } else {
    const int64_t slot = partial_slot(it.slot_base, it.tile_splits, kvh, it.split, lr);
    float* pp = a.part_o + slot * D + 4 * hf;
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i;
        *reinterpret_cast<f32x4*>(pp + db * 32 + i * 8) =
            f32x4{acc[db][r] * inv_l, acc[db][r + 1] * inv_l, acc[db][r + 2] * inv_l, acc[db][r + 3] * inv_l};
      }
    if (hf == 0) a.part_lse2[slot] = lse2;
  }
}

template <int D, bool FP8>
hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  using G = Geometry<D>;
  const size_t lds = (size_t)G::kBytesK + G::kBytesV + (size_t)a.page_slots * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static int lds_opt_in = 0;  // largest dynamic LDS size requested so far
  if ((int)lds > lds_opt_in) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, FP8>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_opt_in = (int)lds;
  }
  dim3 grid((unsigned)a.num_items, (unsigned)a.num_kv_heads);
  hipLaunchKernelGGL((prefill_kernel<D, FP8>), grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int kv_dtype, hipStream_t stream) {
  const bool fp8 = kv_dtype == 1;
  if (head_dim == 128) return fp8 ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
  if (head_dim == 256) return fp8 ? launch_one<256, true>(a, stream) : launch_one<256, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dpp
