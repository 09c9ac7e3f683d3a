// Causal GQA prefill attention over a paged KV cache, gfx950 (CDNA4), wave64.
//
// One workgroup = one (q tile, KV split, kv head). Each wave owns 32 packed rows as two 16-row
// MFMA column blocks; 8 waves (two per SIMD, 256-row tiles) at head_dim 128, 4 waves (one per
// SIMD, 128-row tiles) at head_dim 256. Per KV tile of BN keys (64 at head_dim 128, 32 at
// head_dim 256; tiles start at absolute multiples of BN):
//   gather   every thread loads 16-byte chunks of K and V rows through the page table into
//            registers, PF tiles ahead, then stores them into two LDS stages (natural
//            [key][d] layout, 16-byte chunks XOR-swizzled by key). Keys past kv_len or on an
//            out-of-range page are zero-filled; fp8 E4M3 chunks are decoded to bf16 on the way.
//   QK^T     S^T[key, row] = K Q^T on v_mfma_f32_16x16x32_bf16, fp32 accumulation over
//            head_dim in ascending 32-wide chunks: keys on M, 16 query rows on N, so a lane
//            holds scores of a single query row (4 keys of every 16-key block).
//   mask     keys past the row's position p = kv_len - qo_len + token get -inf (a select after
//            identical arithmetic; tiles wholly below the diagonal skip the select, which
//            would change no bit there).
//   softmax  online, fp32, base 2, with a lazily moved reference max r (c = sm_scale log2 e):
//            t = c max_j s_j; if t > r + 8 then r' = t, alpha = exp2(r - r') else r' = r,
//            alpha = 1; P_j = exp2(fma(s_j, c, -r')) (so P_j <= 2^8); l = fma(l, alpha, sum_j P_j);
//            O = alpha O. Row max and row sum: one fixed pairwise tree over the lane's values,
//            then a butterfly over the four lanes holding the row.
//   PV       O^T[d, row] = alpha O^T + V^T P^T on the same MFMA, P rounded to bf16 (RNE). The
//            V^T operand comes straight from the natural layout through ds_read_tr16_b64.
// After a split's last tile a row writes o = O / l (bf16) and lse = (r + log2 l) ln 2, or, if
// its keys reach past one 4096-token split, the split's fp32 partial (O / l, r + log2 l).
//
// Why this is batch invariant: a row's bits depend on its query, keys 0..p, the tile and split
// grid (absolute positions), the MFMA shapes and the code above -- not on which tile, wave or
// lane holds it, how many rows share its tile, or what else is in the batch. Rows never mix in
// an MFMA column, every lane runs the same reduction trees, the reference max follows the row's
// own scores, and a tile past a row's position is an exact no-op for it (alpha = 1, P = 0, V
// zero-filled past kv_len), so a wave may skip such tiles. The sglang PR #46351 page ("Root cause") shows FlashInfer losing this by
// sizing its q tile from the batch's average query length; here no launch choice enters the
// arithmetic.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "dpp_internal.h"
#include "kernels.h"

namespace dpp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define DPP_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309417f;
// Rebase threshold of the online softmax's reference max, in log2 units (P_j <= 2^8).
constexpr float kRebase = 8.0f;

template <int D>
struct Cfg {
  static constexpr int THREADS = 64 * waves_for(D);
  static constexpr int BM = block_m_for(D);        // packed query rows per tile
  static constexpr int BN = block_n_for(D);        // keys per KV tile
  static constexpr int CH = D / 8;                 // 16-byte bf16 chunks per K/V row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // one of K or V, bf16
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int NS = 2;                     // LDS stages (one barrier per tile)
  static constexpr int CPT = BN * CH / THREADS;    // chunks per thread per tensor per tile
  static constexpr int KB = BN / 16;               // 16-key blocks (QK M blocks)
  static constexpr int DC = D / 32;                // 32-wide head_dim chunks (QK k-steps)
  static constexpr int DB = D / 16;                // 16-wide head_dim blocks (PV M blocks)
  static constexpr int KC = BN / 32;               // 32-key chunks (PV k-steps)
  static constexpr int RPW = rows_per_wave_for(D);  // packed rows per wave
  static constexpr int NB = RPW / 16;              // 16-row column blocks per wave
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
  static_assert(CPT * THREADS == BN * CH, "staging covers the tile");
  static_assert(CH >= 16, "swizzle needs 16 chunks per row");
  static_assert(KC >= 1 && KB == 2 * KC, "tile shape");
};

// Byte offset of 16-byte chunk c of key row `key` inside the K tile. The XOR with key % 16
// spreads the 16 key rows one QK^T operand read touches (same chunk) over all banks.
template <int ROW_BYTES>
__device__ inline int chunk_off(int key, int c) {
  return key * ROW_BYTES + ((c ^ (key & 15)) << 4);
}
// Same for the V tile, swizzled in 32-byte units: a transposing read takes 32 bytes from each
// of 4 consecutive keys per 16 lanes (8 keys per 32 lanes), which this spreads over all banks.
template <int ROW_BYTES>
__device__ inline int chunk_off_v(int key, int c) {
  return key * ROW_BYTES + ((c ^ ((key & 7) << 1)) << 4);
}

// OCP E4M3 code -> fp32 (exact): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
// S.1111.111 is NaN, no infinities.
__device__ inline float e4m3_to_f32(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t em = code & 0x7Fu;
  if (em == 0x7Fu) return __uint_as_float(0x7FC00000u | sign);
  if (em < 8u) return __uint_as_float(sign | __float_as_uint((float)em * 0.001953125f));
  return __uint_as_float(sign | ((em + (120u << 3)) << 20));
}

// Two fp32 -> two bf16, round to nearest even, in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 8 E4M3 codes -> 8 bf16, value = decode(code) * scale (exact for power-of-two scales).
__device__ inline u32x4 dequant8(u32x2 raw, float scale) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t x = raw[w];
    out[2 * w] = pack_bf16x2(e4m3_to_f32(x & 0xFFu) * scale, e4m3_to_f32((x >> 8) & 0xFFu) * scale);
    out[2 * w + 1] = pack_bf16x2(e4m3_to_f32((x >> 16) & 0xFFu) * scale, e4m3_to_f32(x >> 24) * scale);
  }
  return out;
}

template <bool FP8>
struct Raw;
template <>
struct Raw<false> {
  u32x4 v;
};
template <>
struct Raw<true> {
  u32x2 v;
};

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Butterfly over the four lanes (l, l^16, l^32, l^48) holding one query row, on the gfx950
// lane-swap instructions: permlane16_swap(x, x) hands every lane the pair {x[l & ~16],
// x[l | 16]} and permlane32_swap(x, x) the pair {x[l & 31], x[(l & 31) + 32]}, always in that
// order, so each lane of a row combines the same operands in the same order and ends with the
// same bits: ((x0 + x1) + (x2 + x3)) for the sum.
__device__ inline float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, bool FP8, int PF>
__global__ __launch_bounds__(64 * waves_for(D), 1) void prefill_kernel(PrefillArgs a) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int64_t* pg_lds = reinterpret_cast<int64_t*>(smem + C::LDS_BYTES);  // page byte offsets, -1 = bad id

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  const int kvh = blockIdx.y;

  const HeaderPreamble* pre = reinterpret_cast<const HeaderPreamble*>(a.header);
  if (pre->magic != kHeaderMagic || pre->plan_id != a.plan_id) return;  // not this plan's work list
  const PrefillItem it =
      reinterpret_cast<const PrefillItem*>(a.header + pre->item_offset)[a.item_begin + blockIdx.x];
  const RequestDesc rq = reinterpret_cast<const RequestDesc*>(a.header + pre->request_offset)[it.request];

  const int g = a.group;
  const int tile_rows = min(C::BM, rq.qo_len * g - it.row_start);
  const int ctx = rq.kv_len - rq.qo_len;  // position of query token 0
  const int lg = lane >> 4;                // 16-lane group: 8-wide k slice in, 4 output rows out
  const int li = lane & 15;                // column (query row) within a 16-row block
  const int split_key0 = it.split * kSplitTokens;

  // Rows of this lane: tile-local packed row lr = 32*wave + 16*nb + li.
  int p_row[C::NB];    // position of the row (INT_MAX past the tile: no key is masked)
  int nb_pmax[C::NB];  // wave-uniform: largest position among the block's valid rows, -1 if none
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int lr0 = wave * C::RPW + nb * 16;
    const int lr = lr0 + li;
    p_row[nb] = lr < tile_rows ? ctx + (it.row_start + lr) / g : INT_MAX;
    nb_pmax[nb] = lr0 < tile_rows ? ctx + (it.row_start + min(lr0 + 15, tile_rows - 1)) / g : -1;
  }
  const int p_min = ctx + it.row_start / g;
  int wave_pmax = -1;  // largest position among the wave's valid rows
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) wave_pmax = max(wave_pmax, nb_pmax[nb]);

  // ---- page ids of the keys this item visits -> LDS
  const int page_size = a.page_size;
  const int page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz(page_size) : -1;
  const int key_lo = it.kv_tile_begin * C::BN;
  const int key_hi = min(it.kv_tile_end * C::BN, rq.kv_len);
  const int key_lo_page = key_lo / page_size;
  const int n_pages = key_hi > key_lo ? (key_hi - 1) / page_size - key_lo_page + 1 : 0;
  constexpr int kElemBytes = FP8 ? 1 : 2;
  const int64_t token_bytes = (int64_t)a.num_kv_heads * D * kElemBytes;
  const int64_t page_bytes = token_bytes * page_size;
  for (int i = tid; i < n_pages; i += C::THREADS) {
    const int64_t id = a.kv_indices[rq.page_start + key_lo_page + i];
    pg_lds[i] = (id >= 0 && id < a.num_pages) ? id * page_bytes : -1;
  }

  // ---- query rows as the QK^T B operand: lane (lg, li) holds head_dim [32dc + 8lg, +8)
  bf16x8 qreg[C::NB][C::DC];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int lr = wave * C::RPW + nb * 16 + li;
    const bool valid = lr < tile_rows;
    const int R = it.row_start + lr;
    const int token = R / g;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(rq.q_start + token) * a.num_qo_heads + kvh * g + (R - token * g)) * D + 8 * lg;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4*>(qp + dc * 32);
      qreg[nb][dc] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();  // page table visible

  // ---- staging: this thread moves chunks q = tid + THREADS*i (key q / CH, chunk q % CH)
  Raw<FP8> kst[PF][C::CPT], vst[PF][C::CPT];

  // Branch-free gather (a branch around each load would keep the compiler from counting
  // outstanding loads, and it would then wait for every prefetched tile at each LDS store):
  // a chunk past kv_len, or on a page id outside the pool, reads 16 zero bytes from the
  // preamble's reserved words instead. When the page size is a power of two no larger than
  // a KV tile, a thread's page slot and in-page offset are the same for every tile.
  const unsigned char* zero16 = reinterpret_cast<const unsigned char*>(pre->reserved);
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k_pool);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v_pool);
  const bool pow2_pages = page_shift >= 0 && page_size <= C::BN;
  int kr[C::CPT];          // key row of the tile this thread stages
  int pg_rel[C::CPT];      // its page, relative to the tile's first page (pow2_pages)
  int64_t in_page[C::CPT]; // byte offset inside the page: slot, kv head, chunk
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int q = tid + C::THREADS * i;
    kr[i] = q / C::CH;
    const int64_t chunk_bytes = ((int64_t)kvh * D + (q % C::CH) * 8) * kElemBytes;
    pg_rel[i] = pow2_pages ? (kr[i] >> page_shift) : 0;
    in_page[i] = (pow2_pages ? (int64_t)(kr[i] & (page_size - 1)) * token_bytes : 0) + chunk_bytes;
  }
  auto load_tile = [&](int slot, int kt) {
    const int tile_page = pow2_pages ? ((kt * C::BN) >> page_shift) - key_lo_page : 0;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int j = kt * C::BN + kr[i];
      int64_t off;
      if (pow2_pages) {
        off = pg_lds[tile_page + pg_rel[i]];
        off = off < 0 ? off : off + in_page[i];
      } else {
        const int jj = min(j, rq.kv_len - 1);
        const int pi = jj / page_size;
        const int64_t po = pg_lds[pi - key_lo_page];
        off = po < 0 ? po : po + (int64_t)(jj - pi * page_size) * token_bytes + in_page[i];
      }
      const bool ok = j < rq.kv_len && off >= 0;
      const unsigned char* kp = ok ? kbase + off : zero16;
      const unsigned char* vp = ok ? vbase + off : zero16;
      if constexpr (FP8) {
        kst[slot][i].v = *reinterpret_cast<const u32x2*>(kp);
        vst[slot][i].v = *reinterpret_cast<const u32x2*>(vp);
      } else {
        kst[slot][i].v = *reinterpret_cast<const u32x4*>(kp);
        vst[slot][i].v = *reinterpret_cast<const u32x4*>(vp);
      }
    }
  };

  auto store_tile = [&](int slot, int stage) {
    unsigned char* kt_lds = smem + stage * C::STAGE_BYTES;
    unsigned char* vt_lds = kt_lds + C::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int q = tid + C::THREADS * i;
      const int off = chunk_off<C::ROW_BYTES>(q / C::CH, q % C::CH);
      const int off_v = chunk_off_v<C::ROW_BYTES>(q / C::CH, q % C::CH);
      if constexpr (FP8) {
        *reinterpret_cast<u32x4*>(kt_lds + off) = dequant8(kst[slot][i].v, a.k_scale);
        *reinterpret_cast<u32x4*>(vt_lds + off_v) = dequant8(vst[slot][i].v, a.v_scale);
      } else {
        *reinterpret_cast<u32x4*>(kt_lds + off) = kst[slot][i].v;
        *reinterpret_cast<u32x4*>(vt_lds + off_v) = vst[slot][i].v;
      }
    }
  };

  // ---- online-softmax state of this lane's rows
  const float c = a.scale_log2;
  float m_sc[C::NB], l_sum[C::NB];  // reference max (scaled, base 2) and running sum per row
  f32x4 acc[C::DB][C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    m_sc[nb] = -INFINITY;
    l_sum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int kt0 = it.kv_tile_begin;
  const int kt1 = it.kv_tile_end;
  // Tile T lives in register slot (T - kt0) % PF until it is stored into LDS stage
  // (T - kt0) % NS. Prologue: tiles kt0 .. kt0+PF-1 in flight, tile kt0 stored, its slot
  // refilled with tile kt0+PF. Loads are issued unconditionally (tile numbers past the end
  // re-read the last tile, which is never stored): with every load on every path the
  // compiler can wait for exactly one tile at each store instead of for all of them.
  const int kt_last = kt1 - 1;
#pragma unroll
  for (int s = 0; s < PF; ++s) load_tile(s, min(kt0 + s, kt_last));
  store_tile(0, 0);
  load_tile(0, min(kt0 + PF, kt_last));
  __syncthreads();

  // Per tile: store tile kt+1 into its stage (that stage was last read two tiles ago, before
  // the previous barrier), refill the freed slot with tile kt+1+PF, compute tile kt, barrier.
  // Unrolled by PF so every register slot index is a compile-time constant.
  for (int base = kt0; base < kt1; base += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kt = base + u;
      const bool live = kt < kt1;  // the last unrolled group may run past the item's tiles
      const int rel = kt - kt0;
      if (kt + 1 < kt1) store_tile((u + 1) % PF, (rel + 1) % C::NS);
      load_tile((u + 1) % PF, min(kt + 1 + PF, kt_last));

      const unsigned char* k_lds = smem + (rel % C::NS) * C::STAGE_BYTES;
      const unsigned char* v_lds = k_lds + C::TILE_BYTES;
      const int key0 = kt * C::BN;
      const bool diag = key0 + C::BN - 1 > p_min;

      // The wave has work in this tile when one of its valid rows reaches key0. Its blocks
      // then all run the same straight-line code: for a row that does not reach key0 every
      // score is masked, alpha = 1 and P = 0, so the tile changes none of its state.
      if (live && wave_pmax >= key0) {
        // S^T = K Q^T
        f32x4 s[C::KB][C::NB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) s[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < C::DC; ++dc) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(k_lds + chunk_off<C::ROW_BYTES>(kb * 16 + li, dc * 4 + lg));
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
              s[kb][nb] = mfma16(ka, qreg[nb][dc], s[kb][nb]);
          }
        }
        // causal mask: s[kb][nb][j] holds key key0 + 16kb + 4lg + j of row p_row[nb]
        if (diag) {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) {
            const int thr = p_row[nb] - key0 - 4 * lg;  // masked iff 16kb + j > thr
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
              for (int j = 0; j < 4; ++j) s[kb][nb][j] = (kb * 16 + j > thr) ? -INFINITY : s[kb][nb][j];
          }
        }
        // online softmax, per 16-row block
        bf16x8 pb[C::KC][C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          float mx = s[0][nb][0];
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[kb][nb][j]);
          mx = row_max4(mx);
          // The reference max moves only when this tile's max exceeds it by more than
          // kRebase (and on the row's first keys); otherwise P_j <= 2^kRebase and O, l keep
          // their scale. Same softmax, and O is rescaled only on the rare rebase.
          const float mx_sc = mx * c;
          const bool rebase = mx_sc > m_sc[nb] + kRebase;
          const float m_use = rebase ? mx_sc : m_sc[nb];
          const float alpha = rebase ? __builtin_amdgcn_exp2f(m_sc[nb] - m_use) : 1.f;
          m_sc[nb] = m_use;
          float pv[C::KB][4];
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[kb][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][nb][j], c, -m_use));
          // row sum: pairs within each 4-key group, then a pairwise tree over the groups
          float t[C::KB];
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) t[kb] = (pv[kb][0] + pv[kb][1]) + (pv[kb][2] + pv[kb][3]);
#pragma unroll
          for (int w = C::KB / 2; w >= 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
          const float rs = row_sum4(t[0]);
          l_sum[nb] = __builtin_fmaf(l_sum[nb], alpha, rs);
          if (__any(rebase)) {  // acc * 1 == acc for the lanes that keep their reference
#pragma unroll
            for (int db = 0; db < C::DB; ++db) acc[db][nb] *= alpha;
          }
          // P^T as the PV B operand: k = 8lg + t is key 32kc + 16(t/4) + 4lg + t%4
#pragma unroll
          for (int kc = 0; kc < C::KC; ++kc) {
            const u32x4 w4 = u32x4{pack_bf16x2(pv[2 * kc][0], pv[2 * kc][1]),
                                   pack_bf16x2(pv[2 * kc][2], pv[2 * kc][3]),
                                   pack_bf16x2(pv[2 * kc + 1][0], pv[2 * kc + 1][1]),
                                   pack_bf16x2(pv[2 * kc + 1][2], pv[2 * kc + 1][3])};
            pb[kc][nb] = __builtin_bit_cast(bf16x8, w4);
          }
        }
        // O^T += V^T P^T. V^T comes transposed from the natural layout: lane (lg, r) of read h
        // points at key 32kc + 16h + 4lg + r/4, head_dim 16db + 4(r%4), and receives
        // V[32kc + 16h + 4lg + j][16db + li] for j = 0..3 -- the A operand's k = 8lg + 4h + j.
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
#pragma unroll
          for (int kc = 0; kc < C::KC; ++kc) {
            s16x4 hv[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int key = kc * 32 + h * 16 + lg * 4 + (li >> 2);
              const int e = db * 16 + 4 * (li & 3);
              const unsigned char* addr = v_lds + chunk_off_v<C::ROW_BYTES>(key, e >> 3) + (e & 7) * 2;
              hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DPP_LDS s16x4*)(addr));
            }
            const s16x8 v8 = __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
              acc[db][nb] = mfma16(va, pb[kc][nb], acc[db][nb]);
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds O^T[d = 16db + 4lg + j][row 16nb + li]
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int lr = wave * C::RPW + nb * 16 + li;
    const int p = p_row[nb];
    if (lr >= tile_rows || p < split_key0) continue;  // not a row of this split
    const int R = it.row_start + lr;
    const int token = R / g;
    const float inv_l = 1.f / l_sum[nb];
    const float lse2 = m_sc[nb] + __builtin_amdgcn_logf(l_sum[nb]);
    if (p / kSplitTokens == 0) {
      const int64_t orow = (int64_t)(rq.q_start + token) * a.num_qo_heads + kvh * g + (R - token * g);
      uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + orow * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        *reinterpret_cast<u32x2*>(op + db * 16) =
            u32x2{pack_bf16x2(acc[db][nb][0] * inv_l, acc[db][nb][1] * inv_l),
                  pack_bf16x2(acc[db][nb][2] * inv_l, acc[db][nb][3] * inv_l)};
      if (lg == 0) a.lse[orow] = lse2 * kLn2;
    } else {
      const int64_t slot = partial_slot(it.slot_base, it.tile_splits, kvh, it.split, lr, C::BM);
      float* pp = a.part_o + slot * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        *reinterpret_cast<f32x4*>(pp + db * 16) =
            f32x4{acc[db][nb][0] * inv_l, acc[db][nb][1] * inv_l, acc[db][nb][2] * inv_l, acc[db][nb][3] * inv_l};
      if (lg == 0) a.part_lse2[slot] = lse2;
    }
  }
}

template <int D, bool FP8, int PF>
hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  using C = Cfg<D>;
  const size_t lds = (size_t)C::LDS_BYTES + (size_t)a.page_slots * 8;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static int lds_opt_in = 0;  // largest dynamic LDS size requested so far
  if ((int)lds > lds_opt_in) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, FP8, PF>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_opt_in = (int)lds;
  }
  dim3 grid((unsigned)a.num_items, (unsigned)a.num_kv_heads);
  hipLaunchKernelGGL((prefill_kernel<D, FP8, PF>), grid, dim3(C::THREADS), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int kv_dtype, hipStream_t stream) {
  const bool fp8 = kv_dtype == 1;
  if (head_dim == 128) return fp8 ? launch_one<128, true, 2>(a, stream) : launch_one<128, false, 2>(a, stream);
  if (head_dim == 256) return fp8 ? launch_one<256, true, 2>(a, stream) : launch_one<256, false, 2>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dpp
