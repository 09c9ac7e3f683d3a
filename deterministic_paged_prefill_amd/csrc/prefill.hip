// Causal GQA prefill attention over a paged KV cache, gfx950 (CDNA4), wave64.
//
// A unit = one (q tile, KV split, kv head); a workgroup runs one unit, or in a persistent
// launch a chain of units. 8 waves, two per SIMD: each wave owns 32 packed rows as two
// 16-row MFMA column blocks at head_dim 64 and 128 (256-row tiles), one 16-row block at 256
// (128-row tiles); at head_dim 512, 4 waves of one block (64-row tiles). Per KV tile of BN
// keys (64 at head_dim <= 128, 32 above; tiles start at absolute multiples of BN):
//   gather   16-byte chunks of K and V rows come through the page table straight into a ring
//            of four K and four V LDS buffers (two of each at head_dim 512) by LDS-DMA,
//            several tiles ahead (natural
//            [key][d] layout, 16-byte chunks XOR-swizzled by key). Keys past kv_len or on an
//            out-of-range page read zeros; fp8 E4M3 chunks go through registers and are
//            decoded to bf16 on the way.
//   QK^T     S^T[key, row] = K Q^T on v_mfma_f32_16x16x32_bf16, fp32 accumulation over
//            head_dim in ascending 32-wide chunks: keys on M, 16 query rows on N, so a lane
//            holds scores of a single query row (4 keys of every 16-key block).
//   mask     keys past the row's position p = kv_len - qo_len + token get -inf (a select after
//            identical arithmetic; tiles wholly below the diagonal skip the select, which
//            would change no bit there).
//   softmax  online, fp32, base 2, with a lazily moved reference max r (c = sm_scale log2 e):
//            t = c max_j s_j; if t > r + 8 then r' = t, alpha = exp2(r - r') else r' = r,
//            alpha = 1; P_j = exp2(fma(s_j, c, -r')) (so P_j <= 2^8); O = alpha O. Row max: a
//            fixed max3 chain over the lane's values, then a butterfly over the four lanes
//            holding the row. Row sum: each of the four lanes keeps its own share,
//            l_lane = fma(l_lane, alpha, pairwise tree of its P_j); after the split's last
//            tile l = (l_0 + l_1) + (l_2 + l_3) by the same butterfly.
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

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <type_traits>

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
#define DPP_GLOBAL __attribute__((address_space(1)))

constexpr float kLn2 = 0.693147180559945309417f;
// Rebase threshold of the online softmax's reference max, in log2 units (P_j <= 2^8).
constexpr float kRebase = 8.0f;
// LDS operand reads of QK^T and PV run this many MFMA steps ahead of their use: a step is
// NB MFMAs, so a wave with one 16-row block reads further ahead.
template <int NB>
constexpr int ahead_for() { return NB == 1 ? 7 : 3; }

// BNX: keys per KV tile. block_n_for(D) in every batch-invariant plan; a plan in the
// adaptive-tile comparison mode runs narrow tiles with 32 keys at D = 128.
template <int D, int NB, int BNX = block_n_for(D)>
struct Geo {
  static constexpr int WAVES = waves_for(D);
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int PLAN_BM = block_m_for(D);   // packed rows of a planned q tile
  static constexpr int RPW = 16 * NB;              // rows this instantiation gives a wave
  static constexpr int BN = BNX;                   // keys per KV tile
  static constexpr int CH = D / 8;                 // 16-byte bf16 chunks per K/V row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // one KV tile of K or V in bf16
  static constexpr int NBUF = ring_buffers_for(D);  // LDS buffers per tensor (4, or 2 at D = 512)
  static constexpr int KB = BN / 16;               // 16-key blocks (QK M blocks)
  static constexpr int DC = D / 32;                // 32-wide head_dim chunks (QK k-steps)
  static constexpr int DB = D / 16;                // 16-wide head_dim blocks (PV M blocks)
  static constexpr int KC = BN / 32;               // 32-key chunks (PV k-steps)
  static constexpr int NCH = BN * CH / THREADS;    // 16-byte chunks per thread per tensor per tile
  static constexpr int KPI = 64 * 16 / ROW_BYTES;  // key rows one wave-wide DMA load covers
  static constexpr int LDS_BYTES = 2 * NBUF * TILE_BYTES;
  static_assert(BN != block_n_for(D) || LDS_BYTES == ring_bytes_for(D), "ring size");
  // narrow bf16 kernel: P^T and alpha of two tiles, then l and m, passed between two waves
  static constexpr int XSLOT = 64 * KC * 16 + 64 * 4;
  static constexpr int XBYTES = 2 * XSLOT + 2 * 64 * 4;
  static_assert(NCH * THREADS == BN * CH, "the threads cover a tile");
  static_assert(NCH * 64 * WAVES * 16 == TILE_BYTES, "one DMA load per wave moves 1 KiB");
  static_assert(RPW * WAVES >= kNarrowRows && RPW * WAVES <= PLAN_BM, "tile rows fit the waves");
  static_assert(CH >= 8, "swizzles need 8 chunks per row");
  static_assert(KC >= 1 && KB == 2 * KC, "tile shape");
};

// K tile: 16-byte chunk c of key row `key` sits at chunk c ^ kswz(key). The XOR with key % 16
// (key % 8 for 128-byte rows, head_dim 64) spreads the key rows one QK^T operand read touches
// (same chunk) over the banks.
template <int ROW_BYTES>
__device__ constexpr int kswz(int key) {
  return key & ((ROW_BYTES / 16 < 16 ? ROW_BYTES / 16 : 16) - 1);
}
template <int ROW_BYTES>
__device__ inline int chunk_off(int key, int c) {
  return key * ROW_BYTES + ((c ^ kswz<ROW_BYTES>(key)) << 4);
}
// V tile, swizzled in 32-byte units: a transposing read takes 32 bytes from each of 4
// consecutive keys per 16 lanes (8 keys per 32 lanes). Rows of 256 bytes or more move unit u
// to u ^ (key % 8); rows of 128 bytes (head_dim 64, or half of head_dim 128 with VH) to
// u ^ ((key / 2) % 4), so the 8 keys of a half-wave land on 8 distinct 32-byte bank groups.
template <int ROW_BYTES>
__device__ constexpr int vswz(int key) {
  static_assert(ROW_BYTES >= 128, "V rows of at least 128 bytes");
  return ROW_BYTES >= 256 ? (key & 7) << 1 : ((key >> 1) & 3) << 1;
}
template <int ROW_BYTES>
__device__ inline int chunk_off_v(int key, int c) {
  return key * ROW_BYTES + ((c ^ vswz<ROW_BYTES>(key)) << 4);
}

// Two fp32 -> two bf16, round to nearest even, in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 8 OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; S.1111.111 is NaN,
// no infinities) -> 8 bf16, value = decode(code) * scale. v_cvt_pk_f32_fp8 decodes two codes of
// a word exactly to fp32 (every E4M3 value is an fp32 value); the product is rounded to bf16
// (exact for power-of-two scales).
__device__ inline u32x4 dequant8(u32x2 raw, float scale) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[w], false);  // codes in bytes 0, 1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[w], true);   // bytes 2, 3
    out[2 * w] = pack_bf16x2(lo[0] * scale, lo[1] * scale);
    out[2 * w + 1] = pack_bf16x2(hi[0] * scale, hi[1] * scale);
  }
  return out;
}

// The same for a power-of-two scale in [2^-64, 2^64]: v_cvt_scalef32_pk_bf16_fp8 decodes two
// codes and applies the scale's exponent in one instruction. Every product is then an exact
// normal bf16 (an E4M3 value has 4 significant bits, exponents -9..8), so the bits equal
// dequant8's (checked on the GPU for all 256 codes at several scales).
__device__ inline u32x4 dequant8_pow2(u32x2 raw, float scale) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    out[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], scale, false));
    out[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], scale, true));
  }
  return out;
}

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Maximum of two scores (never NaN) as one instruction: fmaxf would first quiet each operand
// it cannot prove canonical (max(x, x)), which is every value from a lane swap.
__device__ inline float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Butterfly over the four lanes (l, l^16, l^32, l^48) holding one query row, on the gfx950
// lane-swap instructions: permlane16_swap(x, x) hands every lane the pair {x[l & ~16],
// x[l | 16]} and permlane32_swap(x, x) the pair {x[l & 31], x[(l & 31) + 32]}, always in that
// order, so each lane of a row combines the same operands in the same order and ends with the
// same bits: ((x0 + x1) + (x2 + x3)) for the sum.
__device__ inline float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One LDS-DMA load: each lane of the wave fetches 16 bytes from its own global address and
// lane l's bytes land at LDS byte address lds_base + 16 l. The LDS address goes in M0, one
// wait state before the load. Issued as assembly so that the compiler does not count it
// among its own outstanding loads (it would otherwise wait for every DMA load in flight at
// each barrier); the kernel waits for its DMA loads itself with wait_vmcnt.
__device__ inline void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(lds_base)
               : "memory");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A wave-uniform 64-bit value held in scalar registers (the inline assembly below takes its
// descriptors in scalar registers).
__device__ inline uint64_t uniform64(uint64_t x) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32)) << 32);
}

// Raw buffer descriptor (stride 0: num_records counts bytes) over [base, base + bytes); a
// load at an offset past `bytes` returns zeros.
__device__ inline i32x4 buffer_rsrc(uint64_t base, uint32_t bytes) {
  return i32x4{(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

// LDS-DMA through a buffer descriptor: lane l fetches 16 bytes at descriptor offset
// voff (zeros past num_records) and they land at LDS byte address lds_base + 16 l.
__device__ inline i32x4 uniform_rsrc(i32x4 r) {
  return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
// (rsrc and lds_base are wave-uniform; readfirstlane only states it to the compiler)
__device__ inline void dma16_buf(int voff, i32x4 rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// Same with 4 bytes a lane, landing at lds_base + 4 l.
__device__ inline void dma4_buf(int voff, i32x4 rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// s_waitcnt vmcnt(N), no wait on the other counters.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// How a chunk's global address is found (a template parameter, fixed per launch):
//   kPagesGeneral  any page size: per-lane division by page_size
//   kPagesPow2     page_size a power of two no larger than a KV tile: a chunk's page within
//                  its tile and its offset in that page are the same for every tile
//   kPagesScalar   page_size a power of two holding whole wave-wide loads (a multiple of the
//                  keys one load covers): the page of a load is uniform, its address is built
//                  as a buffer descriptor in scalar registers whose size ends at kv_len (the
//                  hardware returns zeros past it); bf16 loads are LDS-DMA, fp8 loads go to
//                  registers
//   kPagesScalarDiv the same for any other page size holding whole loads (page and row of a
//                  key by division)
//   kPagesOff32    kPagesPow2's per-lane pages, for a pool of at most 4 GiB: one buffer
//                  descriptor per tensor and unit, and a 32-bit offset per lane (past kv_len or
//                  on an invalid page an offset past the descriptor's range, which reads zeros)
constexpr int kPagesGeneral = 0, kPagesPow2 = 1, kPagesScalar = 2, kPagesScalarDiv = 3, kPagesOff32 = 4;

// NB: 16-row blocks per wave. VH (narrow bf16 kernel only): the launch runs every unit on two
// workgroups, one per half of head_dim in PV. Both compute the unit's scores and softmax from
// all of K; each loads only its half of V's columns and writes its half of the output. Every
// output element still accumulates the same MFMA sequence, so the bits are those of one
// workgroup; the unit's bytes per workgroup drop to 3/4 and twice the workgroups stream them.
// NARROW: the instantiation for passes of tiles with at most kNarrowRows rows (NB = 1).
template <int D, bool FP8, int NB, bool NARROW, int MODE, bool VH, int BNX>
__global__ __launch_bounds__(64 * waves_for(D), 1) void prefill_kernel(PrefillArgs a) {
  using C = Geo<D, NB, BNX>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Narrow bf16 kernel with eight waves: wave 0 computes scores and softmax, wave 4 (on the
  // same SIMD) the output, and waves 2, 3, 6, 7 issue the DMA loads.
  static_assert(!NARROW || NB == 1, "a narrow tile is one 16-row block");
  constexpr bool kSpec = !FP8 && NARROW && waves_for(D) == 8;
  constexpr bool kScalar = MODE == kPagesScalar || MODE == kPagesScalarDiv;  // buffer descriptors
  static_assert(!VH || (kSpec && !kScalar), "head_dim halves: narrow bf16 kernel, vector addresses");
  // V ring: rows of head_dim (or of half of it, VH) per tile
  constexpr int VROW = VH ? C::ROW_BYTES / 2 : C::ROW_BYTES;
  constexpr int VTILE = VH ? C::TILE_BYTES / 2 : C::TILE_BYTES;
  constexpr int RING = C::NBUF * (C::TILE_BYTES + VTILE);
  constexpr int VDB = VH ? C::DB / 2 : C::DB;  // PV head_dim blocks of this workgroup
  // Two-group schedule (see below): bf16 wide tiles with two waves per SIMD. Its launches may
  // be persistent (a chain of units per workgroup).
  constexpr bool kPP = !FP8 && !NARROW && C::WAVES == 8 && NB * 16 == rows_per_wave_for(D);
  unsigned char* xb = smem + RING;  // exchange buffer (kSpec)
  // page-id tables after the ring: raw ids from kv_indices, 4 bytes an entry; a persistent
  // launch alternates between two (the next unit's ids load during the current unit)
  unsigned char* pt0 = xb + (kSpec ? C::XBYTES : 0);
  const int pt_bytes = (int)page_table_bytes(a.page_slots, D);
  int32_t* pg_lds = reinterpret_cast<int32_t*>(pt0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  constexpr int kElem = FP8 ? 1 : 2;

  // ---- the unit (item, kv head) record: word k in lane k of one register, read into scalar
  // registers by decode. A persistent launch starts workgroup b at record b of its chain
  // records; otherwise work w = kvh * num_items + item goes to block b (which the dispatcher
  // hands to XCD b % kXcds): in a wide launch the planner's block table names it (each pair
  // of XCDs a contiguous range of w of equal cost, longest units first; a block without a
  // unit exits at once), in a narrow one w = xcd_chunked(b, n) (each XCD one contiguous range
  // of equal count). Contiguous ranges keep the q tiles that read one request's KV for one kv
  // head, and the two workgroups of a head_dim-split unit, on few L2s.
  const HeaderPreamble* pre = reinterpret_cast<const HeaderPreamble*>(a.header);
  const bool chained = a.chain_offset >= 0;
  auto fetch_record = [&](int idx) -> int32_t {
    const int32_t* r = a.header + a.chain_offset + idx * kItemWords;
    return lane < kItemWords ? r[lane] : 0;
  };
  int32_t rv;
  int vh = 0;  // VH: the half of head_dim this workgroup's PV covers (uniform)
  if (chained) {
    rv = fetch_record(blockIdx.x);
  } else {
    // VH: the two workgroups of a unit are work indices 2u and 2u + 1, so that both usually
    // fall in one XCD's range and share its L2 for K
    const int nw = a.num_items * a.num_kv_heads;
    int w;
    if (!VH && a.block_table >= 0) {
      w = a.header[a.block_table + blockIdx.x];
      if (w < 0 || w >= nw) return;  // no unit for this block (uniform: before any wait)
    } else {
      w = xcd_chunked(blockIdx.x, VH ? 2 * nw : nw);
    }
    if constexpr (VH) {
      vh = w & 1;
      w >>= 1;
    }
    const int h = w / a.num_items;
    const int32_t* r = a.header + a.item_offset + (a.item_begin + (w - h * a.num_items)) * kItemWords;
    rv = lane < kItemWords ? r[lane] : 0;
    rv = lane == 7 ? -1 : (lane == 12 ? h : rv);  // the unit record's next and kv_head words
  }
  const uint32_t magic = pre->magic, plan_id = pre->plan_id;  // one round trip for both
  if ((magic != kHeaderMagic) | (plan_id != a.plan_id)) return;  // not this plan's work list
  auto decode = [&](int32_t v) {
    UnitRecord u;
    u.request = __builtin_amdgcn_readlane(v, 0);
    u.row_start = __builtin_amdgcn_readlane(v, 1);
    u.split = __builtin_amdgcn_readlane(v, 2);
    u.tile_splits = __builtin_amdgcn_readlane(v, 3);
    u.kv_tile_begin = __builtin_amdgcn_readlane(v, 4);
    u.kv_tile_end = __builtin_amdgcn_readlane(v, 5);
    u.slot_base = __builtin_amdgcn_readlane(v, 6);
    u.next = __builtin_amdgcn_readlane(v, 7);
    u.req.q_start = __builtin_amdgcn_readlane(v, 8);
    u.req.qo_len = __builtin_amdgcn_readlane(v, 9);
    u.req.page_start = __builtin_amdgcn_readlane(v, 10);
    u.req.kv_len = __builtin_amdgcn_readlane(v, 11);
    u.kv_head = __builtin_amdgcn_readlane(v, 12);
    u.block = u.pass = u.pad = 0;
    return u;
  };

  const int g = a.group;
  const int lg = lane >> 4;                // 16-lane group: 8-wide k slice in, 4 output rows out
  const int li = lane & 15;                // column (query row) within a 16-row block
  const int row_wave = kSpec ? 0 : wave;  // whose 16-row blocks this wave works on
  // Packed row R = R0 + off of a wave (R0 = the tile's first row + RPW * row_wave, 0 <= off <
  // RPW) is token t0 + q of q head h0 + off - q g, with (t0, h0) = divmod(R0, g) once per
  // unit and q = (h0 + off) / g taken as (h0 + off) * ceil(2^24 / g) >> 24. That quotient is
  // exact while (h0 + off) * g < 2^24, which g <= 1024 (checked by the planner) keeps.
  const uint32_t g_magic = ((1u << 24) + (uint32_t)g - 1u) / (uint32_t)g;
  struct RowPos {
    int token, head;  // token of the request's query, q head within the kv head's group
  };
  auto row_base = [&](int row_start) {  // (t0, h0) of this wave's rows of a tile at row_start
    const int r0 = row_start + row_wave * C::RPW;
    const int t0 = r0 / g;
    return RowPos{t0, r0 - t0 * g};
  };
  auto row_pos = [&](RowPos b, int off) {
    const int x = b.head + off;
    const int q = (int)(((uint32_t)x * g_magic) >> 24);
    return RowPos{b.token + q, x - q * g};
  };
  const int page_size = a.page_size;
  const int page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz(page_size) : -1;
  // page of a key and the key's row in it (scalar page modes)
  auto page_of = [&](int key) {
    if constexpr (MODE == kPagesScalarDiv) return key / page_size;
    else return key >> page_shift;
  };
  auto row_in_page = [&](int key) {
    if constexpr (MODE == kPagesScalarDiv) return key % page_size;
    else return key & (page_size - 1);
  };
  const int64_t token_bytes = (int64_t)a.num_kv_heads * D * kElem;
  const int64_t page_bytes = token_bytes * page_size;

  // ---- state of the current unit
  int kvh, cur_next;
  PrefillItem it;
  RequestDesc rq;
  int tile_rows, ctx, p_min, kt0, n_tiles, key_lo_page, n_pages;
  bool has_rows, s_rows, o_rows;
  int p_row[NB];  // position of the lane's rows (INT_MAX past the tile: no key is masked)
  const unsigned char* kbase;  // the unit's kv head inside the K and V pools
  const unsigned char* vbase;
  // pages [lo, lo + n) of request u.req hold keys [kv_tile_begin BN, min(kv_tile_end BN, kv_len))
  auto page_span = [&](const UnitRecord& u, int& lo, int& n) {
    const int key_lo = u.kv_tile_begin * C::BN;
    const int key_hi = min(u.kv_tile_end * C::BN, u.req.kv_len);
    lo = key_lo / page_size;
    n = key_hi > key_lo ? (key_hi - 1) / page_size - lo + 1 : 0;
  };
  auto set_unit = [&](const UnitRecord& u) {
    kvh = u.kv_head;
    cur_next = u.next;
    it.request = u.request;
    it.row_start = u.row_start;
    it.split = u.split;
    it.tile_splits = u.tile_splits;
    it.kv_tile_begin = u.kv_tile_begin;
    it.kv_tile_end = u.kv_tile_end;
    it.slot_base = u.slot_base;
    rq = u.req;
    tile_rows = min(C::PLAN_BM, rq.qo_len * g - it.row_start);
    ctx = rq.kv_len - rq.qo_len;  // position of query token 0
    has_rows = row_wave * C::RPW < tile_rows;  // wave-uniform
    s_rows = has_rows && (!kSpec || wave == 0);  // scores and softmax
    o_rows = has_rows && (!kSpec || wave == 4);  // output
    // Rows of this lane: tile-local packed row lr = RPW*wave + 16*nb + li.
    const RowPos rb = row_base(it.row_start);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lr = row_wave * C::RPW + nb * 16 + li;
      p_row[nb] = lr < tile_rows ? ctx + row_pos(rb, nb * 16 + li).token : INT_MAX;
    }
    p_min = ctx + it.row_start / g;
    kt0 = it.kv_tile_begin;
    n_tiles = it.kv_tile_end - kt0;  // >= 1
    page_span(u, key_lo_page, n_pages);
    // ragged KV: the request's keys start at its first token (page_start), on page id 0
    const int64_t base_off = (int64_t)kvh * D * kElem + (a.ragged ? (int64_t)rq.page_start * token_bytes : 0);
    kbase = reinterpret_cast<const unsigned char*>(a.k_pool) + base_off;
    vbase = reinterpret_cast<const unsigned char*>(a.v_pool) + base_off;
  };
  UnitRecord first = decode(rv);
  set_unit(first);

  // ---- page ids of a unit -> LDS table, by DMA (lane l of load c brings entry 64c + l;
  // entries past the unit's pages read as 0 and are never used)
  auto load_page_ids = [&](const UnitRecord& u, int32_t* table) {
    int lo, n;
    page_span(u, lo, n);
    // (ragged: one entry, read from the zero chunk a.kv_indices then points at)
    const uint64_t src = reinterpret_cast<uint64_t>(a.kv_indices + (a.ragged ? 0 : u.req.page_start) + lo);
    const i32x4 rsrc = buffer_rsrc(uniform64(src), (uint32_t)__builtin_amdgcn_readfirstlane(n * 4));
    const uint32_t t0 = (uint32_t)(uintptr_t)table;
    for (int c = wave; c * 64 < n; c += C::WAVES) dma4_buf((c * 64 + lane) * 4, rsrc, t0 + (uint32_t)c * 256u);
  };
  load_page_ids(first, pg_lds);

  // ---- query rows as the QK^T B operand: lane (lg, li) holds head_dim [32dc + 8lg, +8)
  bf16x8 qreg[NB][C::DC];
  auto load_q = [&]() {
    const RowPos rb = row_base(it.row_start);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lr = row_wave * C::RPW + nb * 16 + li;
      const bool valid = lr < tile_rows && s_rows;
      const RowPos rp = row_pos(rb, nb * 16 + li);
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           ((int64_t)(rq.q_start + rp.token) * a.num_qo_heads + kvh * g + rp.head) * D + 8 * lg;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(qp + dc * 32);
        qreg[nb][dc] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  // Q of another unit of the chain (a persistent workgroup loads the next unit's Q during its
  // current unit's last A phase, once the last QK^T has read the registers)
  auto load_q_of = [&](const UnitRecord& u) {
    const int u_rows = min(C::PLAN_BM, u.req.qo_len * g - u.row_start);
    const bool w_rows = row_wave * C::RPW < u_rows;  // has_rows of that unit
    const RowPos rb = row_base(u.row_start);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lr = row_wave * C::RPW + nb * 16 + li;
      const bool valid = lr < u_rows && w_rows;
      const RowPos rp = row_pos(rb, nb * 16 + li);
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           ((int64_t)(u.req.q_start + rp.token) * a.num_qo_heads + u.kv_head * g + rp.head) * D +
                           8 * lg;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(qp + dc * 32);
        qreg[nb][dc] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  if constexpr (!kPP) {
    load_q();
    // Q and the page ids in registers and LDS before any DMA load of K or V is issued: a wait
    // for them inside the loop would also wait for every DMA load in flight
    wait_vmcnt<0>();
    __syncthreads();  // page table visible
  }

  // ---- gather. Chunk i (0 <= i < NCH) of this thread in every KV tile is a fixed 16-byte
  // piece of a fixed key row; only the page it sits on changes from tile to tile. A chunk
  // past kv_len, of a tile outside the item, or on a page id outside the pool reads 16 zero
  // bytes from the preamble's zero chunk instead: the loads never branch, so their
  // number per tile is fixed.
  //   bf16: the chunks of one wave's DMA load are the 64 consecutive LDS chunks
  //         [64 (i WAVES + wave), +64); the global chunk is chosen so that it lands in its
  //         swizzled slot.
  //   fp8:  chunk q = tid + THREADS i, loaded to registers, decoded, stored to its slot.
  constexpr bool pow2_pages = MODE != kPagesGeneral;
  constexpr bool kLanePow2 = MODE == kPagesPow2 || MODE == kPagesOff32;  // per-lane, power-of-two pages
  // (fp8 with scalar pages: register loads through buffer descriptors, see fp8_load)
  // Waves that issue DMA loads: 2, 3, 6, 7 in the narrow bf16 kernel, otherwise all.
  constexpr int IW = kSpec ? 4 : C::WAVES;
  const int iw = kSpec ? ((wave & 1) | ((wave >> 2) << 1)) : wave;  // index among the issuers
  const bool issuer = !kSpec || (wave & 2) != 0;
  constexpr int NL = C::TILE_BYTES / (IW * 1024);         // their loads per tensor per tile
  constexpr int NCHT = FP8 ? C::NCH : NL;                 // chunks per thread per tensor per tile
  constexpr int KA = kPP ? 3 : C::NBUF;                   // load group t brings K(t + KA), V(t + VA)
  constexpr int VA = C::NBUF - 2;
  const unsigned char* zero16 = reinterpret_cast<const unsigned char*>(pre->zero_chunk);
  int krow[NCHT];        // key row inside the tile
  int kcol[NCHT];        // byte offset of the K chunk inside the kv head's part of a token row
  int vcol[NCHT];        // same for V
  int lds_k[NCHT];       // fp8: LDS byte offset of the decoded K chunk (V: lds_v)
  int lds_v[NCHT];
  int pg_rel[NCHT];      // pow2 pages: page of the key row relative to the tile's first
  int64_t in_page[NCHT]; // pow2 pages: byte offset of the key row inside its page
#pragma unroll
  for (int i = 0; i < NCHT; ++i) {
    int c_k, c_v;
    if constexpr (FP8) {
      const int q = tid + C::THREADS * i;
      krow[i] = q / C::CH;
      c_k = c_v = q % C::CH;
      lds_k[i] = chunk_off<C::ROW_BYTES>(krow[i], c_k);
      lds_v[i] = chunk_off_v<C::ROW_BYTES>(krow[i], c_v);
    } else {
      const int q = (i * IW + iw) * 64 + lane;
      krow[i] = q / C::CH;
      const int slot = q % C::CH;
      c_k = slot ^ kswz<C::ROW_BYTES>(krow[i]);  // chunk_off(key, c_k) == 16 q
      c_v = slot ^ vswz<C::ROW_BYTES>(krow[i]);  // chunk_off_v(key, c_v) == 16 q
      lds_k[i] = lds_v[i] = 0;
    }
    kcol[i] = c_k * 8 * kElem;
    vcol[i] = c_v * 8 * kElem;
    pg_rel[i] = kLanePow2 ? (krow[i] >> page_shift) : 0;
    in_page[i] = kLanePow2 ? (int64_t)(krow[i] & (page_size - 1)) * token_bytes : 0;
  }
  // V chunks: the same as K's, or, VH, the chunks of this workgroup's half rows (8 key rows
  // of 128 bytes per wave-wide load at D = 128)
  constexpr int NCHV = VH ? NCHT / 2 : NCHT;
  static_assert(FP8 || NCHV * IW * 1024 == VTILE, "the issuing waves cover a V tile");
  int vrow[NCHV], vcolh[NCHV], vpg_rel[NCHV];
  int64_t vin_page[NCHV];
#pragma unroll
  for (int i = 0; i < NCHV; ++i) {
    if constexpr (VH) {
      const int q = (i * IW + iw) * 64 + lane;
      constexpr int HCH = C::CH / 2;
      vrow[i] = q / HCH;
      const int slot = q % HCH;
      vcolh[i] = (vh * HCH + (slot ^ vswz<VROW>(vrow[i]))) * 8 * kElem;  // chunk_off_v<VROW>(.) == 16 q
    } else {
      vrow[i] = krow[i];
      vcolh[i] = vcol[i];
    }
    vpg_rel[i] = kLanePow2 ? (vrow[i] >> page_shift) : 0;
    vin_page[i] = kLanePow2 ? (int64_t)(vrow[i] & (page_size - 1)) * token_bytes : 0;
  }
  // scalar pages: byte offset of the lane's chunk from its load's first key row
  int voff_k[NCHT], voff_v[NCHT];
#pragma unroll
  for (int i = 0; i < NCHT; ++i) {
    voff_k[i] = (int)((krow[i] % C::KPI) * token_bytes) + kcol[i];
    voff_v[i] = (int)((krow[i] % C::KPI) * token_bytes) + vcol[i];
  }
  // source of a chunk (key row `row` of the tile, byte column `col`) of item tile t of one tensor
  auto chunk_src = [&](const unsigned char* base, int col, int row, int t) -> const unsigned char* {
    const int kt = kt0 + min(max(t, 0), n_tiles - 1);
    const int key = kt * C::BN + row;
    int64_t pid, inpg;
    if constexpr (MODE == kPagesPow2) {
      pid = pg_lds[((kt * C::BN) >> page_shift) - key_lo_page + (row >> page_shift)];
      inpg = (int64_t)(row & (page_size - 1)) * token_bytes;
    } else {
      const int kk = min(key, rq.kv_len - 1);
      const int pi = kk / page_size;
      pid = pg_lds[pi - key_lo_page];
      inpg = (int64_t)(kk - pi * page_size) * token_bytes;
    }
    const bool ok = t >= 0 && t < n_tiles && key < rq.kv_len && pid >= 0 && pid < a.num_pages;
    return ok ? base + (pid * page_bytes + inpg + col) : zero16;
  };

  // LDS: K buffers 0..NBUF-1, then V buffers 0..NBUF-1; tile t uses buffers t % NBUF.
  // Load group t brings K(t + NBUF) and V(t + NBUF - 2). It is issued in iteration t and
  // complete before the barrier that ends iteration t + NBUF - 2; iteration t reads K(t + 1)
  // and V(t - 1). K(t + NBUF) replaces K(t), last read in iteration t - 1 (K(0): in the
  // prologue, which ends with a barrier for it), and V(t + NBUF - 2) replaces V(t - 2), last
  // read in iteration t - 1. With two buffers (head_dim 512) a group is complete within its own
  // iteration; the narrow two-wave and two-group schedules are built for four.
  static_assert(C::NBUF == 4 || (C::NBUF == 2 && !kSpec && !kPP), "ring depth of the schedules");
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;  // LDS byte address of the dynamic block
  // LDS byte offset of ring buffer t of K or V
  auto kbuf_off = [&](int t) { return (t & (C::NBUF - 1)) * C::TILE_BYTES; };
  auto vbuf_off = [&](int t) { return C::NBUF * C::TILE_BYTES + (t & (C::NBUF - 1)) * VTILE; };
  // N chunks of tile t: key rows, page of the row within its tile, offset in the page, column
  auto dma_chunks = [&](const unsigned char* base, uint32_t buf, int t, const auto& rows, const auto& pgr,
                        const auto& inp, const auto& cols) {
    constexpr int N = std::extent<std::remove_reference_t<decltype(rows)>>::value;
    if constexpr (pow2_pages) {
      // all page ids first (one LDS round trip), then selects: no branch per chunk
      const bool tile_ok = t >= 0 && t < n_tiles;
      const int kt = kt0 + min(max(t, 0), n_tiles - 1);
      const int lim = tile_ok ? rq.kv_len - kt * C::BN : 0;  // key row r exists iff r < lim
      const int tp = ((kt * C::BN) >> page_shift) - key_lo_page;
      int32_t pid[N];
#pragma unroll
      for (int i = 0; i < N; ++i) pid[i] = pg_lds[tp + pgr[i]];
      if constexpr (MODE == kPagesOff32) {
        // the tensor's descriptor from this kv head's base over the rest of the pool
        const i32x4 rsrc = buffer_rsrc(uniform64(reinterpret_cast<uint64_t>(base)),
                                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(a.pool_bytes - (uint32_t)(kvh * D * kElem))));
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const bool ok = rows[i] < lim && pid[i] >= 0 && pid[i] < a.num_pages;
          const uint32_t off = (uint32_t)pid[i] * (uint32_t)page_bytes + (uint32_t)inp[i] + (uint32_t)cols[i];
          dma16_buf((int)(ok ? off : 0xFFFFFFF0u), rsrc, buf + (uint32_t)((i * IW + iw) * 1024));
        }
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const bool ok = rows[i] < lim && pid[i] >= 0 && pid[i] < a.num_pages;
          const uint64_t off = (uint64_t)(uint32_t)(ok ? pid[i] : 0) * (uint64_t)page_bytes +
                               (uint64_t)inp[i] + (uint64_t)cols[i];
          dma16(ok ? base + off : zero16, buf + (uint32_t)((i * IW + iw) * 1024));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) dma16(chunk_src(base, cols[i], rows[i], t), buf + (uint32_t)((i * IW + iw) * 1024));
    }
  };
  auto dma_tile = [&](bool v, int t) {
    if constexpr (kScalar) {
      // scalar pages are issued by issue_group_scalar
    } else if (v) {
      dma_chunks(vbase, lds0 + (uint32_t)vbuf_off(t), t, vrow, vpg_rel, vin_page, vcolh);
    } else {
      dma_chunks(kbase, lds0 + (uint32_t)kbuf_off(t), t, krow, pg_rel, in_page, kcol);
    }
  };
  u32x2 kreg[C::NCH], vreg[C::NCH];  // fp8 staging of one load group
  // fp8 with scalar pages (a power-of-two page size holding the K8 = 64 / CH key rows of one
  // wave's load): load i of this wave covers rows [r0(i), r0(i) + K8) of its tile, one page,
  // so it reads through a buffer descriptor (uniform) at a per-lane offset; keys past kv_len
  // and pages outside the pool read zeros by the descriptor's range. The 2 NCH descriptors of
  // a group are computed one per lane (lane j: load j, K for j < NCH) and moved to scalar
  // registers with readlane; lane j reads its page id from the LDS table one group ahead.
  constexpr int K8 = 64 / C::CH;
  constexpr int kLoads8 = 2 * C::NCH;
  const int l8 = min(lane, kLoads8 - 1);
  const bool l8_v = l8 >= C::NCH;
  const int l8_r0 = ((64 * wave + C::THREADS * (l8_v ? l8 - C::NCH : l8)) / C::CH);  // r0 of the lane's load
  const int voff8 = (lane / C::CH) * (int)token_bytes + (lane % C::CH) * 8;
  int32_t id8 = 0;  // page id of this lane's load of the next group
  auto read_ids8 = [&](int tk, int tv) {
    const int kt = kt0 + min(max(l8_v ? tv : tk, 0), n_tiles - 1);
    id8 = pg_lds[min(page_of(kt * C::BN + l8_r0) - key_lo_page, n_pages - 1)];
  };
  auto fp8_load_scalar = [&](int tk, int tv) {
    const int t = l8_v ? tv : tk;
    const bool good = id8 >= 0 && id8 < a.num_pages;
    const bool tile_ok = t >= 0 && t < n_tiles;
    const int key0 = (kt0 + min(max(t, 0), n_tiles - 1)) * C::BN + l8_r0;
    const int rows = min(max(rq.kv_len - key0, 0), K8);
    const uint32_t bytes = (tile_ok && good) ? (uint32_t)rows * (uint32_t)token_bytes : 0u;
    const uint64_t addr = reinterpret_cast<uint64_t>(l8_v ? vbase : kbase) +
                          (good ? (uint64_t)(uint32_t)id8 * (uint64_t)page_bytes : 0) +
                          (uint64_t)(uint32_t)(row_in_page(key0) * (int)token_bytes);
#pragma unroll
    for (int j = 0; j < kLoads8; ++j) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)addr, j);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(addr >> 32), j);
      const int nrec = __builtin_amdgcn_readlane((int)bytes, j);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, nrec, 0x00020000);
      const u32x2 val = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff8, 0, 0));
      if (j < C::NCH) kreg[j] = val;
      else vreg[j - C::NCH] = val;
    }
    read_ids8(tk + 1, tv + 1);
  };
  // fp8 with per-lane pages of a pool within 4 GiB: register loads through one descriptor per
  // tensor at a 32-bit offset per lane (past kv_len or on an invalid page: past its range)
  auto fp8_off32 = [&](int col, int row, int t) -> int {
    const int kt = kt0 + min(max(t, 0), n_tiles - 1);
    const int key = kt * C::BN + row;
    const int pid = pg_lds[((kt * C::BN) >> page_shift) - key_lo_page + (row >> page_shift)];
    const bool ok = t >= 0 && t < n_tiles && key < rq.kv_len && pid >= 0 && pid < a.num_pages;
    const uint32_t off = (uint32_t)pid * (uint32_t)page_bytes + (uint32_t)((row & (page_size - 1)) * (int)token_bytes) +
                         (uint32_t)col;
    return (int)(ok ? off : 0xFFFFFFF0u);
  };
  auto fp8_load = [&](int tk, int tv) {
    if constexpr (FP8 && kScalar) {
      fp8_load_scalar(tk, tv);
    } else if constexpr (FP8 && MODE == kPagesOff32) {
      const int nrec = __builtin_amdgcn_readfirstlane((int)(a.pool_bytes - (uint32_t)(kvh * D * kElem)));
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(uniform64(reinterpret_cast<uint64_t>(kbase))), (short)0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(uniform64(reinterpret_cast<uint64_t>(vbase))), (short)0, nrec, 0x00020000);
#pragma unroll
      for (int i = 0; i < C::NCH; ++i) {
        kreg[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, fp8_off32(kcol[i], krow[i], tk), 0, 0));
        vreg[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvs, fp8_off32(vcol[i], krow[i], tv), 0, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::NCH; ++i) {
        kreg[i] = *reinterpret_cast<const u32x2*>(chunk_src(kbase, kcol[i], krow[i], tk));
        vreg[i] = *reinterpret_cast<const u32x2*>(chunk_src(vbase, vcol[i], krow[i], tv));
      }
    }
  };
  auto fp8_store = [&](int tk, int tv) {
    unsigned char* kb = smem + kbuf_off(tk);
    unsigned char* vb = smem + vbuf_off(tv);
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      *reinterpret_cast<u32x4*>(kb + lds_k[i]) =
          a.kv_scale_pow2 ? dequant8_pow2(kreg[i], a.k_scale) : dequant8(kreg[i], a.k_scale);
      *reinterpret_cast<u32x4*>(vb + lds_v[i]) =
          a.kv_scale_pow2 ? dequant8_pow2(vreg[i], a.v_scale) : dequant8(vreg[i], a.v_scale);
    }
  };
  auto issue_group = [&](int t) {  // bf16: DMA of load group t
    dma_tile(false, t + KA);
    dma_tile(true, t + VA);
  };
  // Scalar pages. Load i of this wave in tile t covers key rows [key0, key0 + KPI) of one
  // page, so its address is uniform: a buffer descriptor in scalar registers. The kLoads
  // descriptors of a group are computed side by side, load j in lane j (vector arithmetic,
  // a few instructions for all of them), then moved to scalar registers with readlane; lane j
  // reads its page id from the LDS table one iteration ahead.
  auto page_slot = [&](int t, int i) {
    const int kt = kt0 + min(max(t, 0), n_tiles - 1);
    const int key0 = kt * C::BN + (i * IW + iw) * C::KPI;
    return min(page_of(key0) - key_lo_page, n_pages - 1);
  };
  constexpr int kLoads = 2 * NCHT;
  const int lj = min(lane, kLoads - 1);  // the load this lane prepares (lanes past kLoads: a copy)
  const bool lj_v = lj >= NCHT;          // a V load
  const int lj_i = lj_v ? lj - NCHT : lj;
  int32_t lane_id = 0;  // page id of this lane's load of the next group
  auto read_ids = [&](int g) { lane_id = pg_lds[page_slot(lj_v ? g + VA : g + KA, lj_i)]; };
  // Descriptors of the next group's loads, prepared ahead so that firing a load is an M0
  // write and the load itself.
  struct LoadDesc {
    i32x4 rsrc;
    uint32_t lds;
  };
  LoadDesc nd[kLoads];
  auto prep = [&](int grp) {  // from lane_id (group grp's page ids)
    const int t = lj_v ? grp + VA : grp + KA;
    const int id = lane_id;
    const bool good = id >= 0 && id < a.num_pages;  // else the load reads zeros
    const uint64_t base = reinterpret_cast<uint64_t>(lj_v ? vbase : kbase);
    const bool tile_ok = t >= 0 && t < n_tiles;
    const int key0 = (kt0 + min(max(t, 0), n_tiles - 1)) * C::BN + (lj_i * IW + iw) * C::KPI;
    const uint64_t off = good ? (uint64_t)(uint32_t)id * (uint64_t)page_bytes : 0;
    const int rows = min(max(rq.kv_len - key0, 0), C::KPI);
    const uint32_t bytes = (tile_ok && good) ? (uint32_t)rows * (uint32_t)token_bytes : 0u;
    const uint64_t addr = base + off + (uint64_t)(uint32_t)(row_in_page(key0) * (int)token_bytes);
    const uint32_t lds =
        lds0 + (uint32_t)(((lj_v ? C::NBUF : 0) + (t & (C::NBUF - 1))) * C::TILE_BYTES + (lj_i * IW + iw) * 1024);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)addr, j);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(addr >> 32), j);
      nd[j].rsrc = buffer_rsrc(((uint64_t)hi << 32) | lo, (uint32_t)__builtin_amdgcn_readlane((int)bytes, j));
      nd[j].lds = (uint32_t)__builtin_amdgcn_readlane((int)lds, j);
    }
  };
  auto fire = [&](int j) { dma16_buf(j < NCHT ? voff_k[j] : voff_v[j - NCHT], nd[j].rsrc, nd[j].lds); };
  auto issue_group_scalar = [&](int t) {  // ids hold group t's; then read group t+1's
    prep(t);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) fire(j);
    read_ids(t + 1);
  };
  auto issue = [&](int t) {  // bf16: load group t
    if constexpr (kScalar) issue_group_scalar(t);
    else issue_group(t);
  };
  constexpr int kGroupLoads = kScalar ? kLoads : NCHT + NCHV;  // one thread's loads of a group

  // ---- online-softmax state of this lane's rows
  const float c = a.scale_log2;
  float m_sc[NB], l_sum[NB];  // reference max (scaled, base 2) per row; this lane's share of its sum
  f32x4 acc[VDB][NB];
  auto reset_state = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_sc[nb] = -INFINITY;
      l_sum[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < VDB; ++db) acc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset_state();

  // ---- output of a unit: lane holds O^T[d = 16db + 4lg + j][row 16nb + li]. The unit is
  // given by its record register, so that a wave can write a unit's rows after the next unit
  // has begun.
  // Output pointers as scalar values in the global address space: the two row kinds below
  // store through different pointers under a per-lane condition, and a per-lane choice
  // between two kernel-argument fields would be a per-lane load (whose wait would also wait
  // for every DMA load in flight). Generic pointers would make flat stores, which the LDS
  // counter also tracks: every later LDS wait would wait for them to reach memory.
  DPP_GLOBAL uint16_t* const o_out = (DPP_GLOBAL uint16_t*)uniform64(reinterpret_cast<uint64_t>(a.o));
  DPP_GLOBAL float* const lse_out = (DPP_GLOBAL float*)uniform64(reinterpret_cast<uint64_t>(a.lse));
  DPP_GLOBAL float* const part_o_out = (DPP_GLOBAL float*)uniform64(reinterpret_cast<uint64_t>(a.part_o));
  DPP_GLOBAL float* const part_lse_out = (DPP_GLOBAL float*)uniform64(reinterpret_cast<uint64_t>(a.part_lse2));
  // Rows of the last split (p < 4096) leave as bf16. In the two-group schedule they pass
  // through 2 KiB of LDS per wave (after the page tables; one group writes at a time, beside
  // the other group's loop): 16 rows x 64 head_dim values at a time are written in the MFMA
  // layout and read back as 16-byte pieces of 8 rows, so that every store covers whole
  // 128-byte lines (a store straight from the MFMA layout writes 16 rows x 32 bytes), which
  // the next unit's loads then queue behind for less time. 16-byte chunk c of staged row r
  // sits at chunk c ^ (r % 8). The other schedules end their workgroup with the writes and
  // store straight from the MFMA layout.
  constexpr int kStageBytes = 2048;
  unsigned char* const stage = pt0 + (chained ? 2 : 1) * pt_bytes + (wave & 3) * kStageBytes;
  auto write_out = [&](int32_t rec) {
    const UnitRecord e = decode(rec);
    const int e_rows = min(C::PLAN_BM, e.req.qo_len * g - e.row_start);
    const int e_ctx = e.req.kv_len - e.req.qo_len;
    const int e_key0 = e.split * kSplitTokens;
    const RowPos rb = row_base(e.row_start);
    // output row (in o and lse) of a row at (token, q head)
    auto out_row = [&](RowPos rp) {
      return (int64_t)(e.req.q_start + rp.token) * a.num_qo_heads + e.kv_head * g + rp.head;
    };
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lr = row_wave * C::RPW + nb * 16 + li;  // the row this lane holds
      const RowPos pos = row_pos(rb, nb * 16 + li);
      const int p = lr < e_rows ? e_ctx + pos.token : -1;
      const bool mine = p >= e_key0;                   // a row of this split
      const float l = row_sum4(l_sum[nb]);  // the row's sum from the four lanes' shares
      const float inv_l = 1.f / l;
      const float lse2 = m_sc[nb] + __builtin_amdgcn_logf(l);
      if (mine && p < kSplitTokens) {
        const int64_t orow = out_row(pos);
        if (lg == 0 && vh == 0) lse_out[orow] = lse2 * kLn2;
        if constexpr (!kPP) {
          DPP_GLOBAL uint16_t* op = o_out + orow * D + vh * (D / 2) + 4 * lg;
#pragma unroll
          for (int db = 0; db < VDB; ++db)
            *reinterpret_cast<DPP_GLOBAL u32x2*>(op + db * 16) =
                u32x2{pack_bf16x2(acc[db][nb][0] * inv_l, acc[db][nb][1] * inv_l),
                      pack_bf16x2(acc[db][nb][2] * inv_l, acc[db][nb][3] * inv_l)};
        }
      } else if (mine && e.tile_splits > 1 && e.slot_base >= 0) {
        // a row reaching past the first split: its fp32 partial, straight from the MFMA layout.
        // Only a tile whose last row needs several splits owns a slot block (slot_base >= 0);
        // the planner guarantees p >= 4096 implies that, and the test keeps a slip from writing
        // below the partial region.
        const int64_t slot = partial_slot(e.slot_base, e.tile_splits, e.kv_head, e.split, lr, slot_rows_for(e_rows));
        DPP_GLOBAL float* pp = part_o_out + slot * D + vh * (D / 2) + 4 * lg;
#pragma unroll
        for (int db = 0; db < VDB; ++db)
          *reinterpret_cast<DPP_GLOBAL f32x4*>(pp + db * 16) =
              f32x4{acc[db][nb][0] * inv_l, acc[db][nb][1] * inv_l, acc[db][nb][2] * inv_l, acc[db][nb][3] * inv_l};
        if (lg == 0 && vh == 0) part_lse_out[slot] = lse2;
      }
      if constexpr (kPP) {
        // the two staged rows this lane stores, r = 8h + lane / 8, from 16-byte piece kk
        const int kk = lane & 7;
        int64_t srow[2];
        bool sok[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 8 * h + (lane >> 3);
          const RowPos rp = row_pos(rb, nb * 16 + r);
          const int p_r = row_wave * C::RPW + nb * 16 + r < e_rows ? e_ctx + rp.token : -1;
          sok[h] = p_r >= e_key0 && p_r < kSplitTokens;
          srow[h] = out_row(rp) * D + 8 * kk;
        }
#pragma unroll
        for (int sp = 0; sp < VDB / 4; ++sp) {  // head_dim [64 sp, +64)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int db = 4 * sp + k;
            const int c = (2 * k + (lg >> 1)) ^ (li & 7);
            *reinterpret_cast<DPP_LDS u32x2*>((DPP_LDS unsigned char*)stage + li * 128 + c * 16 + (lg & 1) * 8) =
                u32x2{pack_bf16x2(acc[db][nb][0] * inv_l, acc[db][nb][1] * inv_l),
                      pack_bf16x2(acc[db][nb][2] * inv_l, acc[db][nb][3] * inv_l)};
          }
          asm volatile("" ::: "memory");  // the wave's own LDS writes, then its reads (in order)
          u32x4 v[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = 8 * h + (lane >> 3);
            v[h] = *reinterpret_cast<const DPP_LDS u32x4*>((const DPP_LDS unsigned char*)stage + r * 128 +
                                                           ((kk ^ (r & 7)) << 4));
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (sok[h]) *reinterpret_cast<DPP_GLOBAL u32x4*>(o_out + srow[h] + 64 * sp) = v[h];
          asm volatile("" ::: "memory");
        }
      }
    }
  };

  constexpr int kAhead = ahead_for<NB>();
  constexpr bool kPin = kPP || NB == 1;  // pin the read-ahead order (the scheduler undoes it)
  // S^T = K Q^T for tile t
  auto qk = [&](f32x4 (&s)[C::KB][NB], int t) {
    const unsigned char* k_lds = smem + (t & (C::NBUF - 1)) * C::TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // step st = (dc, kb) with dc outer: every s[kb][nb] accumulates head_dim chunks
    // dc = 0, 1, ... in that order; each step's K operand is read kAhead steps ahead
    constexpr int kS = C::DC * C::KB;
    auto read_k = [&](int st) {
      const int dc = st / C::KB, kb = st % C::KB;
      return *reinterpret_cast<const bf16x8*>(k_lds + chunk_off<C::ROW_BYTES>(kb * 16 + li, dc * 4 + lg));
    };
    bf16x8 ka[kAhead + 1];
#pragma unroll
    for (int st = 0; st < kAhead; ++st) ka[st] = read_k(st);
#pragma unroll
    for (int st = 0; st < kS; ++st) {
      if (st + kAhead < kS) ka[(st + kAhead) % (kAhead + 1)] = read_k(st + kAhead);
      const int dc = st / C::KB, kb = st % C::KB;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[kb][nb] = mfma16(ka[st % (kAhead + 1)], qreg[nb][dc], s[kb][nb]);
      if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);  // keep this order: reads kAhead steps ahead
    }
  };

  // causal mask of tile t: s[kb][nb][j] holds key key0 + 16kb + 4lg + j of row p_row[nb]
  auto mask = [&](f32x4 (&s)[C::KB][NB], int t) {
    const int key0 = (kt0 + t) * C::BN;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int thr = p_row[nb] - key0 - 4 * lg;  // masked iff 16kb + j > thr
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[kb][nb][j] = (kb * 16 + j > thr) ? -INFINITY : s[kb][nb][j];
    }
  };

  // online softmax of one tile: P^T into pb, alpha per row block; returns whether some row
  // of the wave moved its reference (then O must be rescaled by alpha, see rescale)
  auto softmax = [&](f32x4 (&s)[C::KB][NB], bf16x8 (&pb)[C::KC][NB], float (&alpha)[NB],
                     auto rescale_tag) -> bool {
    constexpr bool kRescale = decltype(rescale_tag)::value;  // O lives in this wave
    bool moved = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // the 4 KB scores of the lane's row: max3 over the first three, then two at a time
      // (from -inf, pairwise: max3 instructions with no quieting of the scores)
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4 * C::KB; e += 2)
        mx = fmaxf(fmaxf(mx, s[e / 4][nb][e % 4]), s[(e + 1) / 4][nb][(e + 1) % 4]);
      mx = row_max4(mx);
      // The reference max moves only when this tile's max exceeds it by more than kRebase
      // (and on the row's first keys); otherwise P_j <= 2^kRebase and O, l keep their scale.
      const float mx_sc = mx * c;
      const bool rebase = mx_sc > m_sc[nb] + kRebase;
      const float m_use = rebase ? mx_sc : m_sc[nb];
      alpha[nb] = rebase ? __builtin_amdgcn_exp2f(m_sc[nb] - m_use) : 1.f;
      m_sc[nb] = m_use;
      moved = moved || rebase;
      float pv[C::KB][4];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[kb][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][nb][j], c, -m_use));
      // this lane's share of the row sum: pairs within each 4-key group, then a pairwise tree
      // over the groups
      float ts[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) ts[kb] = (pv[kb][0] + pv[kb][1]) + (pv[kb][2] + pv[kb][3]);
#pragma unroll
      for (int h = C::KB / 2; h >= 1; h >>= 1)
#pragma unroll
        for (int i = 0; i < h; ++i) ts[i] = ts[2 * i] + ts[2 * i + 1];
      l_sum[nb] = __builtin_fmaf(l_sum[nb], alpha[nb], ts[0]);
      if constexpr (kRescale) {
        if (__any(rebase)) {  // acc * 1 == acc for the lanes that keep their reference
#pragma unroll
          for (int db = 0; db < VDB; ++db) acc[db][nb] *= alpha[nb];
        }
      }
      // P^T as the PV B operand: k = 8lg + i is key 32kc + 16(i/4) + 4lg + i%4
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const u32x4 w4 = u32x4{pack_bf16x2(pv[2 * kc][0], pv[2 * kc][1]),
                               pack_bf16x2(pv[2 * kc][2], pv[2 * kc][3]),
                               pack_bf16x2(pv[2 * kc + 1][0], pv[2 * kc + 1][1]),
                               pack_bf16x2(pv[2 * kc + 1][2], pv[2 * kc + 1][3])};
        pb[kc][nb] = __builtin_bit_cast(bf16x8, w4);
      }
    }
    return __any(moved);
  };

  // O^T += V^T P^T for tile t. V^T comes transposed from the natural layout: lane (lg, r) of
  // read h points at key 32kc + 16h + 4lg + r/4, head_dim 16db + 4(r%4), and receives
  // V[32kc + 16h + 4lg + j][16db + li] for j = 0..3 -- the A operand's k = 8lg + 4h + j.
  auto no_hook = [](int) {};
  auto pv_acc = [&](const bf16x8 (&pb)[C::KC][NB], int t, auto&& hook) {
    const unsigned char* v_lds = smem + vbuf_off(t);
    // step st = (kc, db) with kc outer: every acc[db][nb] accumulates key chunks kc = 0, 1,
    // ... in that order; each step's V^T operand is read kAhead steps ahead. With VH, db
    // counts the blocks of this workgroup's half of head_dim.
    constexpr int kS = C::KC * VDB;
    auto read_v = [&](int st) {
      const int kc = st / VDB, db = st % VDB;
      s16x4 hv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = kc * 32 + h * 16 + lg * 4 + (li >> 2);
        const int e = db * 16 + 4 * (li & 3);
        const int off = chunk_off_v<VROW>(key, e >> 3);
        const unsigned char* addr = v_lds + off + (e & 7) * 2;
        hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DPP_LDS s16x4*)(addr));
      }
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 va[kAhead + 1];
#pragma unroll
    for (int st = 0; st < kAhead; ++st) va[st] = read_v(st);
#pragma unroll
    for (int st = 0; st < kS; ++st) {
      if (st + kAhead < kS) va[(st + kAhead) % (kAhead + 1)] = read_v(st + kAhead);
      const int kc = st / VDB, db = st % VDB;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[db][nb] = mfma16(va[st % (kAhead + 1)], pb[kc][nb], acc[db][nb]);
      hook(st);  // work to overlap with this step's MFMAs
      if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);  // keep this order: reads kAhead steps ahead
    }
  };

  // ---- schedule: iteration t = 0 .. n_tiles-1 issues load group t, then (waves with rows)
  // masks S(t) on a diagonal tile, runs PV(t-1) and softmax(t) -- independent matrix-core and
  // vector work, so the wave issues softmax arithmetic while its MFMAs run -- then QK^T(t+1)
  // into the same score registers, and ends with a barrier once load group t-2 has landed.
  // PV(n_tiles-1) follows the loop. Per row this is the plain sequence over tiles:
  // O = alpha(t) O, then O += PV(t). QK^T of the tile past the item reads a zero-filled
  // buffer and is discarded; PV(-1) adds V(-1) P(-1) = 0 * 0 (both zero-filled).
  f32x4 s[C::KB][NB];
  // P^T of the previous tile until PV has issued its MFMAs, then of the current one (the
  // softmax writes it after PV's last read in program order)
  bf16x8 pb[C::KC][NB];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pb[kc][nb] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

  if constexpr (kSpec) {
    // Narrow bf16 kernel: same load schedule as the plain loop below (group t brings K(t+4)
    // and V(t+2), issued in iteration t, landed before the barrier ending iteration t+2).
    // Iteration t: wave 0 masks S(t), runs softmax(t) into P(t) and alpha(t), hands them to
    // wave 4 through LDS slot t&1 and computes QK^T(t+1) into its other score registers;
    // wave 4 takes P(t-1), alpha(t-1) from slot (t-1)&1, rescales O by alpha(t-1) (alpha = 1
    // exactly for the rows that kept their reference) and adds PV(t-1). The two waves share
    // a SIMD, so the softmax arithmetic of one runs beside the MFMAs of the other. Per row
    // the sequence is the plain one: O = alpha(t) O, then O += PV(t). A slot is rewritten
    // two iterations after it was filled, one barrier after wave 4 read it.
    if (issuer) {
      if constexpr (kScalar) {
        read_ids(-C::NBUF);
#pragma unroll
        for (int t = -C::NBUF; t < 0; ++t) issue_group_scalar(t);
      } else {
#pragma unroll
        for (int t = -C::NBUF; t < 0; ++t) issue_group(t);
      }
      wait_vmcnt<2 * kGroupLoads>();  // groups -4 and -3 landed: K(0), K(1), V(-1)
    }
    __syncthreads();
    f32x4 s1[C::KB][NB];
    if (s_rows) qk(s, 0);
    __syncthreads();  // load group 0 overwrites K(0)
    auto put_p = [&](int t, const float (&al)[NB]) {
      unsigned char* slot = xb + (t & 1) * C::XSLOT;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) *reinterpret_cast<bf16x8*>(slot + (kc * 64 + lane) * 16) = pb[kc][0];
      *reinterpret_cast<float*>(slot + 64 * C::KC * 16 + lane * 4) = al[0];
    };
    auto take_p = [&](int t) {  // wave 4: P^T and alpha of tile t, then O = alpha O + PV(t)
      const unsigned char* slot = xb + (t & 1) * C::XSLOT;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) pb[kc][0] = *reinterpret_cast<const bf16x8*>(slot + (kc * 64 + lane) * 16);
      const float al = *reinterpret_cast<const float*>(slot + 64 * C::KC * 16 + lane * 4);
#pragma unroll
      for (int db = 0; db < VDB; ++db) acc[db][0] *= al;
      pv_acc(pb, t, no_hook);
    };
    auto spec_iter = [&](int t, f32x4 (&sc)[C::KB][NB], f32x4 (&sn)[C::KB][NB]) {
      if (issuer) {
        if constexpr (kScalar) issue_group_scalar(t);
        else issue_group(t);
      }
      if (s_rows) {
        if ((kt0 + t) * C::BN + C::BN - 1 > p_min) mask(sc, t);
        float alpha[NB];
        softmax(sc, pb, alpha, std::false_type{});
        put_p(t, alpha);
        if (t + 1 < n_tiles) qk(sn, t + 1);
      }
      if (o_rows && t >= 1) take_p(t - 1);
      if (issuer) wait_vmcnt<2 * kGroupLoads>();  // group t-2 landed
      __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
      spec_iter(t, s, s1);
      if (t + 1 < n_tiles) spec_iter(t + 1, s1, s);
    }
    if (o_rows) take_p(n_tiles - 1);
    // l (lane shares) and m of the rows to wave 4, which writes the outputs
    float* xl = reinterpret_cast<float*>(xb + 2 * C::XSLOT);
    if (s_rows) {
      xl[lane] = l_sum[0];
      xl[64 + lane] = m_sc[0];
    }
    __syncthreads();
    if (o_rows) {
      l_sum[0] = xl[lane];
      m_sc[0] = xl[64 + lane];
    }
  } else if constexpr (!kPP) {
    if constexpr (FP8) {
      if constexpr (kScalar) read_ids8(0, -2);  // the first group's page ids
#pragma unroll
      for (int t = -C::NBUF; t < -1; ++t) {
        fp8_load(t + C::NBUF, t + C::NBUF - 2);
        fp8_store(t + C::NBUF, t + C::NBUF - 2);
      }
      fp8_load(C::NBUF - 1, C::NBUF - 3);  // group -1, stored in iteration 0
    } else {
      if (issuer) {
        if constexpr (kScalar) {
          read_ids(-C::NBUF);
#pragma unroll
          for (int t = -C::NBUF; t < 0; ++t) issue_group_scalar(t);
        } else {
#pragma unroll
          for (int t = -C::NBUF; t < 0; ++t) issue_group(t);
        }
      }
      // groups -NBUF and -NBUF + 1 landed: K(0), K(1), and V(-1) (zeros)
      wait_vmcnt<(C::NBUF - 2) * kGroupLoads>();
    }
    __syncthreads();
    if (has_rows) qk(s, 0);
    // load group 0 overwrites K(0): every wave's QK^T(0) must be done with it first
    if constexpr (!FP8) __syncthreads();

    auto iteration = [&](int t) {
      if constexpr (FP8) {
        fp8_store(t + C::NBUF - 1, t + C::NBUF - 3);  // group t-1
        fp8_load(t + C::NBUF, t + C::NBUF - 2);       // group t
        // with two buffers the tiles just stored, K(t + 1) and V(t - 1), are this iteration's
        if constexpr (C::NBUF == 2) __syncthreads();
      } else if constexpr (kScalar) {
        if (issuer) issue_group_scalar(t);
      } else {
        if (issuer) issue_group(t);
      }
      if (has_rows) {
        if ((kt0 + t) * C::BN + C::BN - 1 > p_min) mask(s, t);
        float alpha[NB];
        pv_acc(pb, t - 1, no_hook);
        softmax(s, pb, alpha, std::true_type{});
        qk(s, t + 1);
      }
      if constexpr (!FP8) wait_vmcnt<(C::NBUF - 2) * kGroupLoads>();  // group t + 2 - NBUF landed
      __syncthreads();
    };
    for (int t = 0; t < n_tiles; ++t) iteration(t);
    if constexpr (FP8 && C::NBUF == 2) {
      // with two buffers the last V tile arrives in group n_tiles - 1, which no iteration stores
      fp8_store(n_tiles + 1, n_tiles - 1);
      __syncthreads();
    }
    if (has_rows) pv_acc(pb, n_tiles - 1, no_hook);
  } else {
    // Two groups: waves 0-3 lead, waves 4-7 (which share the SIMDs with them pairwise) run
    // one phase behind. Per tile t two phases, each closed by a barrier:
    //   B(t)  mask + softmax(t)                                   -- vector ALU
    //   A(t)  PV(t) firing own part of load group t+1, QK^T(t+1)  -- matrix cores
    // so that one wave of a SIMD computes a softmax while the other runs MFMAs. Load group t
    // brings K(t+3) and V(t+2); A(t) reads K(t+1) and V(t), both from group t-2. Every wave
    // waits for its own part of a group before the barrier that opens the leading group's
    // A phase reading it: the leading waves at the end of B(t) for group t-2, the trailing
    // waves (whose B(t) falls in the leading group's A(t)) at the end of their A(t) for
    // group t-1. Group t overwrites K(t-1) and V(t-2), last read by the trailing group's
    // A(t-2), one phase before any wave issues group t (in its A(t-1)). Groups -3..0 are
    // issued up front. Per row the sequence is the plain one: O = alpha(t) O, then
    // O += PV(t).
    //
    // A persistent workgroup runs its chain of units back to back. The leading waves write a
    // unit's rows while the trailing waves run its last PV; the trailing waves write theirs
    // while the next unit's Q and first load group arrive. The next unit's record and page
    // ids are fetched one unit ahead (ids into the other LDS table).
    const bool leading = wave < C::WAVES / 2;
    int tab = 0;  // page table of the current unit
    // records (one word a lane): current unit, the next one, and the one after it (arriving).
    // They move on right after the full wait at the start of a unit, so that no copy of a
    // register still being loaded needs a wait of its own.
    int32_t rcur = rv, rnext = 0, rfetch = 0;
    bool has_prev = false, rotate = false;
    bool q_ready = false;  // this unit's Q was loaded in the previous unit's last A phase
    constexpr bool kLateQ = D <= 128;
    if (cur_next >= 0) rnext = fetch_record(cur_next);
    wait_vmcnt<0>();
    __syncthreads();  // the first unit's page ids visible
    // group g's loads are prepared in B(g-1) and fired between the PV steps of A(g-1)
    constexpr int kEvery = (C::KC * C::DB) / kLoads;
    static_assert(kEvery >= 1, "one load per PV step at most");
    for (;;) {
      // Q (unless loaded ahead) and load group -3 (K(0)). The full wait below covers Q either
      // way. The trailing waves write the previous unit's rows after the barrier, ahead of the
      // next loads: a store counts on the same counter as the loads, so the wait here would
      // hold every wave until the stores are acknowledged, while after the barrier their
      // acknowledgement is due only at the trailing waves' wait for group -2.
      if (!q_ready) load_q();
      q_ready = false;
      if constexpr (kScalar) {
        read_ids(-3);
        issue_group_scalar(-3);
      } else {
        issue(-3);
      }
      wait_vmcnt<0>();
      __syncthreads();
      if (!leading && has_prev) {
        write_out(rcur);  // still the previous unit's record
        reset_state();
      }
      if (rotate) {
        rcur = rnext;
        rnext = rfetch;
      }
      // the next unit's page ids and the record after it (older than the groups below, so the
      // counted waits cover them), then groups -2..0
      const bool has_next = cur_next >= 0;
      if (has_next) {
        const UnitRecord nxt = decode(rnext);
        load_page_ids(nxt, reinterpret_cast<int32_t*>(pt0 + (tab ^ 1) * pt_bytes));
        if (nxt.next >= 0) rfetch = fetch_record(nxt.next);
      }
#pragma unroll
      for (int grp = -2; grp <= 0; ++grp) issue(grp);
      if (has_rows) qk(s, 0);
      if (!leading) {
        wait_vmcnt<2 * kGroupLoads>();  // group -2 (K(1), V(0)) before the leading group's A(0)
        __syncthreads();
      }
      for (int t = 0; t < n_tiles; ++t) {
        if (has_rows) {
          if ((kt0 + t) * C::BN + C::BN - 1 > p_min) mask(s, t);
          float alpha[NB];
          softmax(s, pb, alpha, std::true_type{});
        }
        if constexpr (kScalar) prep(t + 1);
        // A(t) reads group t-2; the leading group's A(t) starts at the next barrier, the
        // trailing group's one phase later (its wait for group t-1 follows its A(t))
        if (leading) wait_vmcnt<2 * kGroupLoads>();
        __syncthreads();
        if constexpr (kScalar) {
          if (has_rows) {
            pv_acc(pb, t, [&](int st) {
              if (st % kEvery == 0 && st / kEvery < kLoads) fire(st / kEvery);
            });
          } else {
#pragma unroll
            for (int j = 0; j < kLoads; ++j) fire(j);
          }
          read_ids(t + 2);
        } else {
          issue(t + 1);
          if (has_rows) pv_acc(pb, t, no_hook);
        }
        if (has_rows && t + 1 < n_tiles) qk(s, t + 1);
        if (t == n_tiles - 1 && has_next && !(kLateQ && leading)) {
          // The last QK^T of this unit ran in A(t-1): its Q registers take the next unit's
          // Q now, in flight during the output write and the transition.
          load_q_of(decode(rnext));
          q_ready = true;
        }
        if (!leading) wait_vmcnt<2 * kGroupLoads>();  // group t-1, for the leading group's A(t+1)
        __syncthreads();
      }
      // the leading waves' rows are final: write them during the trailing group's last A
      if (leading) {
        if (has_rows) write_out(rcur);
        reset_state();
        // At head_dim <= 128 the leading waves load the next unit's Q after their write: a wait
        // for the write's own memory operations (a register reload) would otherwise wait for
        // these loads as well. (At 256 the code generated for that order is slower.)
        if (kLateQ && has_next) {
          load_q_of(decode(rnext));
          q_ready = true;
        }
        __syncthreads();
      }
      if (!has_next) {
        if (!leading && has_rows) write_out(rcur);
        break;
      }
      has_prev = !leading;
      rotate = true;
      set_unit(decode(rnext));
      tab ^= 1;
      pg_lds = reinterpret_cast<int32_t*>(pt0 + tab * pt_bytes);
    }
  }
  wait_vmcnt<0>();  // no load may outlive the workgroup (a DMA load would land in LDS)

  // ---- epilogue (the two-group schedule writes its units' rows inside its chain loop)
  if constexpr (!kPP) {
    if (o_rows) write_out(rv);
  }
}

template <int D, bool FP8, int NB, bool NARROW, int MODE, bool VH = false, int BNX = block_n_for(D)>
hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  using C = Geo<D, NB, BNX>;
  constexpr int kRing = C::NBUF * (C::TILE_BYTES + (VH ? C::TILE_BYTES / 2 : C::TILE_BYTES));
  // page-id tables (4 bytes an entry): a unit's pages plus one tile's worth of slack for the
  // last tile's lookups past kv_len (their chunks read the zero chunk); two in a persistent
  // launch
  constexpr bool kSpec = !FP8 && NARROW && waves_for(D) == 8;
  const size_t pt_bytes = (size_t)page_table_bytes(a.page_slots, D);
  constexpr bool kPP = !FP8 && !NARROW && C::WAVES == 8 && NB * 16 == rows_per_wave_for(D);
  const size_t lds = (size_t)kRing + (kSpec ? C::XBYTES : 0) + (a.chain_offset >= 0 ? 2 : 1) * pt_bytes +
                     (kPP ? (size_t)kOutStageBytes : 0);
  if (lds > (size_t)kLdsLimit) return hipErrorInvalidValue;
  static int lds_opt_in = 0;  // largest dynamic LDS size requested so far
  if ((int)lds > lds_opt_in) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, FP8, NB, NARROW, MODE, VH, BNX>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_opt_in = (int)lds;
  }
  if (VH && a.chain_offset >= 0) return hipErrorInvalidValue;
  if (a.block_table >= 0 && (VH || a.table_blocks < a.num_items * a.num_kv_heads)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.chain_offset >= 0 ? a.num_chains
                       : a.block_table >= 0 ? a.table_blocks
                                            : (VH ? 2 : 1) * a.num_items * a.num_kv_heads));
  if (a.chain_offset >= 0 && !chained_launch(D, FP8, NARROW)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, FP8, NB, NARROW, MODE, VH, BNX>), grid, dim3(C::THREADS), lds, stream, a);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kPersistentBlocks;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = kPersistentBlocks;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int D, int NB, bool NARROW, int BNX = block_n_for(D)>
hipError_t launch_nb(const PrefillArgs& a, bool fp8, hipStream_t stream) {
  const int P = a.page_size;
  const bool pow2 = (P & (P - 1)) == 0;
  if constexpr (BNX == block_n_for(D)) {
    if (fp8) {  // one fp8 schedule: NARROW changes nothing in it
      constexpr int kRowsPerLoad8 = 64 / (D / 8);  // key rows of one wave's fp8 load
      if (pow2 && P >= kRowsPerLoad8) return launch_one<D, true, NB, false, kPagesScalar>(a, stream);
      if (P % kRowsPerLoad8 == 0) return launch_one<D, true, NB, false, kPagesScalarDiv>(a, stream);
      if (pow2 && P <= block_n_for(D) && a.pool_bytes > 0) return launch_one<D, true, NB, false, kPagesOff32>(a, stream);
      return pow2 && P <= block_n_for(D) ? launch_one<D, true, NB, false, kPagesPow2>(a, stream)
                                         : launch_one<D, true, NB, false, kPagesGeneral>(a, stream);
    }
  } else if (fp8) {
    return hipErrorInvalidValue;  // the comparison tile is built for bf16 only
  }
  // The narrow kernel's issuing waves compute nothing else: per-lane (vector) addresses
  // suit them. The wide eight-wave kernel's waves are busy with the softmax: scalar
  // descriptors.
  if constexpr (!NARROW && waves_for(D) == 8) {
    if (pow2 && P >= Geo<D, NB>::KPI) return launch_one<D, false, NB, NARROW, kPagesScalar>(a, stream);
    if (P % Geo<D, NB>::KPI == 0) return launch_one<D, false, NB, NARROW, kPagesScalarDiv>(a, stream);
    // smaller power-of-two pages of a pool within 4 GiB: 32-bit per-lane offsets
    if (pow2 && P <= BNX && a.pool_bytes > 0) return launch_one<D, false, NB, NARROW, kPagesOff32>(a, stream);
  } else if constexpr (NARROW && waves_for(D) == 8 && D >= 128) {
    // A narrow launch of at most one unit per two compute units splits head_dim in PV over
    // two workgroups per unit (same bits). A CU streams a unit's gather at a rate of its own,
    // so two CUs that each load all of K and half of V (3/4 of the unit's bytes) finish sooner
    // than one that loads all of it, while the K they share comes from HBM once.
    if (2 * a.num_items * a.num_kv_heads <= compute_units()) {
      if (pow2 && P <= BNX && a.pool_bytes > 0) return launch_one<D, false, NB, NARROW, kPagesOff32, true, BNX>(a, stream);
      return pow2 && P <= BNX ? launch_one<D, false, NB, NARROW, kPagesPow2, true, BNX>(a, stream)
                              : launch_one<D, false, NB, NARROW, kPagesGeneral, true, BNX>(a, stream);
    }
  }
  if constexpr (NARROW) {
    if (pow2 && P <= BNX && a.pool_bytes > 0) return launch_one<D, false, NB, NARROW, kPagesOff32, false, BNX>(a, stream);
  }
  return pow2 && P <= BNX ? launch_one<D, false, NB, NARROW, kPagesPow2, false, BNX>(a, stream)
                          : launch_one<D, false, NB, NARROW, kPagesGeneral, false, BNX>(a, stream);
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, bool fp8, bool narrow, hipStream_t stream) {
  constexpr int kWide = rows_per_wave_for(D) / 16;
  // four-wave head dims have no narrow specialisation: one instantiation serves both
  constexpr bool kNarrowKernel = waves_for(D) == 8;
  return narrow ? launch_nb<D, 1, kNarrowKernel>(a, fp8, stream) : launch_nb<D, kWide, false>(a, fp8, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int kv_dtype, bool narrow, int block_n,
                          hipStream_t stream) {
  const bool fp8 = kv_dtype == 1;
  if (block_n != block_n_for(head_dim)) {
    // adaptive-tile comparison plans only: narrow bf16 tiles with 32 keys at head_dim 128
    if (head_dim == 128 && block_n == 32 && narrow && !fp8) return launch_nb<128, 1, true, 32>(a, false, stream);
    return hipErrorInvalidValue;
  }
  if (head_dim == 64) return launch_d<64>(a, fp8, narrow, stream);
  if (head_dim == 128) return launch_d<128>(a, fp8, narrow, stream);
  if (head_dim == 256) return launch_d<256>(a, fp8, narrow, stream);
  if (head_dim == 512) return launch_d<512>(a, fp8, narrow, stream);
  return hipErrorInvalidValue;
}

}  // namespace dpp
