// FlashAttention-2 forward kernel for gfx950 (CDNA4), written for wave64 MFMA.
//
// What it computes (per batch b, head h, query row i):
//   O[i]   = sum_j P[i,j] V[j] / l_i,  P[i,j] = exp(scale * q_i.k_j - m_i),
//   l_i    = sum_j P[i,j],             LSE[i] = m_i + ln l_i
// over the keys visible to i: all keys, j <= i (causal), or the keys of a
// sliding window i - wl <= j <= i + wr below a per-sequence key length
// (general mask).  Method:
// "FlashAttention-2 MMA 代码学习" (chuoer47.github.io) step 1 (online (m, l)
// merge over key tiles), step 2 (split-Q: each wave owns whole query rows),
// step 3 (P stays in registers and feeds the second matrix product); and
// "第 15 章 FA2 前向：Tiling 与 Online Softmax" (yangyitao.com) §15.1 (outer loop
// over query tiles, grid over query tile x head x batch, deferred 1/l, LSE
// statistic), §15.3 (skeleton: causal tile bound, ragged-N zero fill and
// -inf column mask, -inf guards, out-of-range rows not stored), §15.5.1
// (K/V tiles staged through shared memory ahead of their use).
//
// gfx950 mapping (a re-design, not a translation of the pages' mma.sync code):
//   * The score tile is computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16}: A = 32 keys x 16 dims (from LDS),
//     B = 16 dims x 32 queries (Q^T, resident in VGPRs for the whole kernel).
//     In the 32x32 accumulator, lane L holds query column L%32 and the 16 keys
//     8*(r/4) + 4*(L/32) + r%4 (r = accumulator register), so a query's row max
//     is an in-lane reduction plus one exchange between the two 32-lane halves
//     (v_permlane32_swap).
//   * The probabilities never leave the lane: registers r = 8u..8u+7 of a
//     32-key accumulator are exactly the B operand (16 keys x 32 queries) of
//     O^T += V^T P^T for k-step u, with keys ordered {16u+4h+e, 16u+8+4h+e}.
//     Their row sums come from a sparse MFMA over the same packed words
//     (tile_sums), so l sums exactly the rounded values the output MFMA uses.
//   * V^T operands come from LDS with ds_read_b64_tr_b16, which transposes a
//     4-row x 16-column block of 16-bit values across 16 lanes; the rows each
//     lane group reads are chosen to match that key order.
//   * Software pipeline inside each wave (run_pipe): sub-iteration j issues the
//     MFMAs of S(j+1) and of P(j-1) V(j-1) one at a time, each followed by a
//     share of the softmax of tile j, so matrix cores and VALU work side by side.
//   * Lazily moved exponent base: the softmax of a tile uses the current base
//     without first taking the tile's max.  Checked form: a tile whose row sums
//     exceed 2^15 (so some probability might overflow 16 bits) goes through
//     the rebase path (row max, rescale O and l, recompute).  Unchecked form
//     (every d but 128 under the general mask): the base stays at the first
//     tile's row max, and a row sum
//     that overflowed sends the whole workgroup through the checked form.  Any
//     base gives the same softmax; the pages move it on every tile.
//   * K and V tiles go from global memory straight into a 4-slot LDS ring
//     (buffer_load ... lds), one barrier per two tiles, with 16-byte-chunk XOR
//     swizzles so the MFMA operand reads do not collide in LDS banks.
//     Out-of-range rows come back as zeros from buffer loads with a
//     range-checked resource (the pages' zero fill), and out-of-range stores
//     are dropped by the same check.
//   * The grid is one workgroup per (query tile, batch*head); consecutive
//     workgroup ids walk the heads first, within groups of heads sized so that
//     an XCD (workgroups are dealt to the 8 XCDs round robin) runs all query
//     tiles of its few heads together and their K/V stay in its L2
//     (work_item).  Causal grids issue the longest query tiles first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Kernel arguments.  All pointers are the base of the full [B,H,N,d] (or
// [B,H,N]) tensor; the kernel offsets them per (batch*head).
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int n;             // sequence length N
  int bh;            // B * H
  int n_qtiles;      // ceil(N / rows per workgroup)
  float scale_log2;  // |scale| * log2(e): scores go to the base-2 exponent domain
  uint32_t q_sign;   // 0x80008000 when scale < 0: Q is negated on load, |scale| used
  // Key j is visible to query i iff j < key_len(b) (every mode) and, under
  // the general mask, j >= i - wl and j <= i + wr (kNoBound: no bound).
  int wl;
  int wr;
  const int* key_lens;  // B lengths (clamped to [0, N]) or null: no padding
  int heads;            // H, to find the batch of a (batch*head) slice
  int group;            // slices per group of the work order (1..bh; see work_item)
};

// Work item of workgroup wg: its (batch*head) slice and its query-tile step
// (the step counts from the longest query tile under a mask, see the
// kernels).  The slices are taken in groups of p.group: every query tile of a
// group comes before the next group, and inside a group the step varies
// slowest and the slice fastest.  Workgroups are dealt to the XCDs round robin
// by index; with p.group a multiple of their count each XCD holds the same
// slices of a group throughout, and a group small enough that its query tiles
// are about one XCD's worth of resident workgroups keeps each slice's
// workgroups walking its keys at nearly the same time, so K and V come from
// that XCD's L2 instead of HBM.  p.group = bh is the plain order (slice
// fastest over all slices).
struct WorkItem {
  int bh;
  int step;
};
__device__ __forceinline__ WorkItem work_item(const Params& p, int wg) {
  const int span = p.group * p.n_qtiles;
  const int g = wg / span;
  const int r = wg - g * span;
  const int size = min(p.group, p.bh - g * p.group);  // the last group may be smaller
  const int step = r / size;
  return {g * p.group + (r - step * size), step};
}

// Mask modes (template argument MASK).
enum : int { kMaskNone = 0, kMaskCausal = 1, kMaskGeneral = 2 };
// A window bound that never hides a key (larger than any N the library
// accepts, small enough that row +- bound stays in int range).
constexpr int kNoBound = 1 << 29;

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle, offsets range-checked against num_records).
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the O and LSE stores of the main kernel (sc0 nt:
// non-temporal, streaming).  Nothing in the launch reads the output again;
// with the whole-row stores of store_output it measured +0.1% to +2.3%
// (the chunked kernel's 8-byte row pieces lose 4.5% with it and keep the
// default).
constexpr int kStreamStore = 3;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// The descriptor make_rsrc builds, as its four dwords: base address (48 bits,
// stride 0), number of bytes, word 3.  Uniform across the wave.
__device__ __forceinline__ u32x4 rsrc_words(const void* tensor, size_t byte_off, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)tensor + byte_off;
  u32x4 w;
  w[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  w[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  w[2] = __builtin_amdgcn_readfirstlane(bytes);
  w[3] = (uint32_t)kRsrcWord3;
  return w;
}

// Values of the pair of lanes L and L^32: (lower-half lane's, upper-half lane's),
// identical in both lanes of the pair.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Output MFMA of the pipelined schedule for head dims of 128 and more: the
// O^T accumulators are kept in AGPRs (only MFMAs and the rare rescale touch
// them), which leaves the arch VGPRs to Q^T, the scores, probabilities and
// LDS fragments.  The compiler does not see inside inline asm: the operands of
// this MFMA are never written by a VALU instruction shortly before it (P is
// packed a whole sub-iteration earlier, O is only rescaled by the rebase path,
// which is followed by softmax work before the next output MFMA), dependent
// MFMAs of one accumulator are always separated by other MFMAs, and the other
// readers of O (the rebase path, the compiler-issued output MFMA of the last
// tile) come after an explicit wait (settle_o).
template <bool BF16>
__device__ __forceinline__ void mfma32_acc_agpr(f32x16& c, const u32x4& a, const u32x4& b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// Sparse 16x16x64 MFMA (A 4:2 structured: two nonzeros in every group of four
// k, their positions given by the index word), used to sum probabilities on
// the matrix cores: c + A B with B the 64 x 16 operand (b0, b1).
template <bool BF16>
__device__ __forceinline__ f32x4 smfmac16(const u32x4& a, const u32x4& b0, const u32x4& b1, const f32x4& c, int idx) {
  const u32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  if constexpr (BF16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, b), c,
                                                     idx, 0, 0);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), c,
                                                    idx, 0, 0);
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> one dword of two 16-bit values, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Design switches.  The library's own build leaves each at its default, the
// shipped design; a build that flips one measures what that choice is worth.
//   FA2_KV_SWIZZLE     1: the K/V chunk permutations below; 0: plain row-major tiles.
//   FA2_KV_SLOTS       4: 4-slot K/V rings, one barrier per 2 tiles; 8: 8 slots
//                      where they fit the LDS, one barrier per 4 tiles; 2: 2
//                      slots, one barrier per tile (the nearest form of a
//                      single K and a single V buffer that this schedule,
//                      which holds K(j+1) and V(j-1) at once, can run).
//   FA2_KV_PAD         0: tiles filled by direct-to-LDS loads into the
//                      swizzled layouts below; 1: tiles loaded into VGPRs and
//                      stored to LDS rows padded by 16 bytes (K) and 64 bytes
//                      (V), no swizzle.
//   FA2_UNCHECKED_RUN  1: fixed-base unchecked first run (not at d = 128
//                      under the general mask);
//                      0: the checked pipeline only.
//   FA2_SPLIT_KV       1: two split-KV wave groups at d = 32 and 64 (host side);
//                      0: one group of 4 waves.
//   FA2_W4_TWO_PER_SIMD 1: the 4-wave forms of d = 64 and of d = 128 with one
//                      query block per wave held to two waves per SIMD (256
//                      registers); 0: no register bound.
//   FA2_XCD_GROUPS     1: slices taken in groups whose query tiles fill one
//                      round of an XCD's resident workgroups (host side, see
//                      work_item); k: k rounds; 0: one group of all slices.
#ifndef FA2_KV_SWIZZLE
#define FA2_KV_SWIZZLE 1
#endif
#ifndef FA2_KV_SLOTS
#define FA2_KV_SLOTS 4
#endif
#ifndef FA2_KV_PAD
#define FA2_KV_PAD 0
#endif
#ifndef FA2_UNCHECKED_RUN
#define FA2_UNCHECKED_RUN 1
#endif
#ifndef FA2_SPLIT_KV
#define FA2_SPLIT_KV 1
#endif
#ifndef FA2_XCD_GROUPS
#define FA2_XCD_GROUPS 1
#endif
#ifndef FA2_W4_TWO_PER_SIMD
#define FA2_W4_TWO_PER_SIMD 1
#endif

// LDS layouts.  A K or V tile is BC rows (keys) of D 16-bit values, stored as
// 16-byte chunks, rows packed back to back; chunk c of row r sits at a
// permuted chunk position of its row.  The gfx950 LDS serves 256 bytes (64
// banks x 4 bytes) per cycle; a 16-byte read by 64 lanes is served 16 lanes
// at a time, so 16 lanes must hit 16 different 16-byte bank groups to go at
// full rate (measured: the rows-only layout runs at a quarter of that).
//  * K rows are read 16 bytes per lane by 32 consecutive rows at one chunk
//    (kslot: position of chunk c in row r).  With 128-byte rows (d = 64) two
//    rows share a 256-byte line, so rows with equal parity need distinct
//    positions: XOR with (r/2)%8.  With 64-byte rows (d = 32) four rows share
//    a line: XOR with (r/4)%4.  With rows of 256 bytes or more every row
//    starts a line: XOR with r%16.  192-byte rows (d = 96) start at bank group
//    12r mod 16, which repeats every 4 rows; an XOR could leave the 12-chunk
//    row, so the chunks rotate by (r/4)%4 instead.  Every rule depends on r
//    only through r%32, which the row offsets added as immediates (multiples
//    of 32 rows) preserve.
//  * V rows are read 8 bytes per lane by ds_read_b64_tr_b16: 32 lanes at a
//    time read 4 consecutive rows 4h+e at 64 bytes (chunks 4b..4b+3) each.
//    With rows of 256 bytes or more the 4 rows meet the same banks (4-way
//    conflicts), with 128-byte rows rows e and e+2 do; XOR chunk bits 2-3 with
//    e (bit 2 with e/2 at d = 64) so the 4 rows fill distinct bank groups.  The
//    swizzle keeps row%4, which the row offsets added as immediates (multiples
//    of 8 rows) preserve.  Measured: 3% faster at d = 256, no change at d = 64
//    and d = 128; the bank-conflict counter of the d = 128 kernel drops to 0.
//    With 64-byte rows (d = 32) the 4 rows fill one line, and with 192-byte
//    rows (d = 96) they start at bank groups 0, 12, 8, 4: no swizzle needed.
template <int D>
__device__ __forceinline__ int kslot(int row, int c) {
  if constexpr (!FA2_KV_SWIZZLE || (FA2_KV_PAD && D <= 128)) return c;
  if constexpr (D == 32) return c ^ ((row >> 2) & 3);
  if constexpr (D == 64) return c ^ ((row >> 1) & 7);
  if constexpr (D == 96) return (c + ((row >> 2) & 3)) % 12;
  return c ^ (row & 15);
}
// Logical chunk stored at position `slot` of row r (the inverse of kslot).
template <int D>
__device__ __forceinline__ int klog(int row, int slot) {
  if constexpr (D == 96 && FA2_KV_SWIZZLE && !FA2_KV_PAD) return (slot + 12 - ((row >> 2) & 3)) % 12;
  return kslot<D>(row, slot);  // the XOR rules are involutions
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (!FA2_KV_SWIZZLE || (FA2_KV_PAD && D <= 128) || D == 32 || D == 96) return 0;
  if constexpr (D == 64) return ((row >> 1) & 1) << 2;
  return (row & 3) << 2;
}

// Per-lane partial row sums of one tile above this value send the tile to the
// rebase path: every probability of the tile is then below it, so it is finite
// and exact to the usual relative rounding in fp16 as well as bf16.
constexpr float kTileSumLimit = 32768.0f;
// Exponent base of a row with no visible key in the first tile of an
// unchecked run: finite (hidden keys still give exp2(-inf) = 0), and so far
// below any score that a visible key overflows the row sum.
constexpr float kUnseenBase = 1.0e30f;

template <int D, int BC, int NW, int QB, int KVG, bool BF16, int MASK>
struct Fa2Fwd {
  static constexpr bool CAUSAL = MASK == kMaskCausal;
  static constexpr bool GENERAL = MASK == kMaskGeneral;
  static_assert(KVG == 1 || (KVG == 2 && NW == 8), "split-KV runs two groups of 4 waves");
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWB = D * 2;             // bytes per K/V row in global memory
  static constexpr int GTILEB = BC * ROWB;       // bytes per K (or V) tile in global memory
  // LDS row strides: rows back to back (the swizzled layouts), or padded
  // rows (FA2_KV_PAD): K + 16 bytes, so that 16 consecutive rows start in 16
  // different 16-byte bank groups, and V + 64 bytes, so that the 4 rows of a
  // transposing read do.  (Padding applies up to d = 128: a padded d = 256 V
  // ring would outgrow the 64 KiB that a ds immediate offset reaches.)
  static constexpr bool KV_PAD = FA2_KV_PAD && D <= 128;
  static constexpr int KROW = KV_PAD ? ROWB + 16 : ROWB;
  static constexpr int VROW = KV_PAD ? ROWB + 64 : ROWB;
  static constexpr int TILEK = BC * KROW;        // LDS bytes per K tile slot
  static constexpr int TILEV = BC * VROW;        // LDS bytes per V tile slot
  // Pipelined schedule: K and V tiles each in a ring of PIPE_RING LDS slots,
  // one barrier per PIPE_RING / 2 sub-iterations.  (An 8-slot ring must fit
  // the 160 KiB LDS and keep each ring within the 64 KiB of ds immediates.)
  static constexpr bool DEEP_RING_FITS =
      8 * TILEK <= 65536 && 8 * TILEV <= 65536 && KVG * 8 * (TILEK + TILEV) <= 160 * 1024;
  static constexpr int PIPE_RING = FA2_KV_SLOTS == 2 ? 2 : (FA2_KV_SLOTS == 8 && DEEP_RING_FITS ? 8 : 4);
  static constexpr int PIPE_G = PIPE_RING / 2;
  static constexpr int QW = 32 * QB;             // query rows per wave
  // KVG = 2 (split-KV): two groups of 4 waves own the same query rows and
  // split the key tiles.  Otherwise all NW waves own rows of their own and
  // share one K/V stream.  With 8 waves every SIMD runs two.
  static constexpr bool SPLIT = KVG == 2;
  static constexpr int QWAVES = SPLIT ? NW / 2 : NW;
  static constexpr int BR = QWAVES * QW;         // query rows per workgroup
  // Threads that stage one K/V stream (split-KV: one stream per group).
  static constexpr int STAGERS = SPLIT ? THREADS / 2 : THREADS;
  static constexpr int STREAMS = SPLIT ? 2 : 1;
  static constexpr int KB = BC / 32;             // 32-key blocks per tile
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  static constexpr int DK = D / 16;              // 16-deep k-steps of S^T = K Q^T
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / STAGERS; // chunks per thread per tile (each of K, V)
  // One K/V stream in LDS: a ring of PIPE_RING tiles each of K and V.
  static constexpr int SLOTS = PIPE_RING;
  static constexpr int STREAMB = SLOTS * (TILEK + TILEV);
  // Split-KV merge area: per group-1 lane, O^T (QB*DB*16 floats) then m, l
  // and the unrounded bf16 row sums.
  static constexpr int MERGE_FLOATS = QB * DB * 16 + 3 * QB;
  static constexpr int MERGE_BYTES = SPLIT ? (NW / 2) * 64 * MERGE_FLOATS * 4 : 0;
  // Output staging (store_output): 32 * QB rows of O per wave; with the
  // split-KV merge, each wave of group 0 in its own merge slot.
  static constexpr int OUT_WAVE_BYTES = 32 * QB * D * 2;
  static constexpr int MERGE_SLOT_BYTES = 64 * MERGE_FLOATS * 4;
  static constexpr int OUT_BYTES = SPLIT ? QWAVES * (MERGE_SLOT_BYTES > OUT_WAVE_BYTES ? MERGE_SLOT_BYTES : OUT_WAVE_BYTES)
                                         : NW * OUT_WAVE_BYTES;
  static constexpr int RING_MERGE_BYTES = STREAMS * STREAMB > MERGE_BYTES ? STREAMS * STREAMB : MERGE_BYTES;
  static constexpr int LDS_BYTES = RING_MERGE_BYTES > OUT_BYTES ? RING_MERGE_BYTES : OUT_BYTES;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BC * CPR) % STAGERS == 0 && CPT >= 1, "staging split");
  // Every LDS access in the tile loop is a lane base register plus a
  // compile-time offset that must fit the instruction's 16-bit immediate; the
  // start of the V ring is kept in the lanes' V offsets, so each ring (K, V)
  // only needs its own 64 KiB of immediates.
  static constexpr int VBASE = SLOTS * TILEK;
  static_assert(STREAMB - VBASE <= 65536 && VBASE <= 65536, "LDS image must fit the ds immediate offset");

  typedef __attribute__((address_space(3))) char lds_char;

  // Lane-constant LDS byte offsets (relative to the K or V buffer base).
  struct LdsOffsets {
    int k[DK];     // K^T operand of k-step ks for key block 0 (block kb adds kb*32 rows)
    int v[DB];     // V^T operand rows 32*db..: keys 4h+e of a 16-key group (+8 rows: second read)
    int vst[CPT];  // store of chunk j through VGPRs, V layout (zeroing a V slot; FA2_KV_PAD: staging)
    int kst[CPT];  // the same, K layout (FA2_KV_PAD: staging)
    int gst[CPT];  // global byte offset of chunk j in row-major order (FA2_KV_PAD)
    int gdk[CPT];  // global byte offset of the K chunk a direct-to-LDS load lands at linear slot j
    int gdv[CPT];  // the same for the V layout
    int dma;       // this wave's first linear slot (bytes) of a direct-to-LDS tile load
  };

  // S^T accumulators of one tile for all query blocks of the wave.
  struct Scores {
    f32x16 s[QB][KB];
  };

  static __device__ __forceinline__ void scores(const lds_char* sk, const LdsOffsets& off,
                                                const u32x4 (&qf)[QB][DK], Scores& out) {
    constexpr int KG = D >= 256 ? 4 : DK;  // K fragments in flight per group
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int g = 0; g < DK; g += KG) {
        u32x4 a[KG];
#pragma unroll
        for (int i = 0; i < KG; ++i) a[i] = *(const __attribute__((address_space(3))) u32x4*)(sk + off.k[g + i] + kb * 32 * KROW);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int i = 0; i < KG; ++i)
            out.s[qb][kb] = mfma32<BF16>(a[i], qf[qb][g + i], (g + i == 0) ? f32x16{} : out.s[qb][kb]);
        }
      }
    }
  }

  // Per-element mask of one tile (ragged tail, causal diagonal, window edges,
  // padding): hidden scores become -inf before the row max, as the pages
  // require.  n: keys present (N, or the sequence's key length).
  static __device__ __forceinline__ void mask_scores(Scores& sc, int lane, int k0, int qw0, int n, int wl,
                                                     int wr) {
    const int half = lane >> 5;
    const float ninf = -__builtin_inff();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + 32 * qb + (lane & 31);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool hide = (key >= n) || (CAUSAL && key > qrow) || (GENERAL && (key > qrow + wr || key < qrow - wl));
          sc.s[qb][kb][r] = hide ? ninf : sc.s[qb][kb][r];
        }
      }
    }
  }

  // O^T += V^T P^T for one V tile in LDS.
  static __device__ __forceinline__ void pv(const lds_char* sv, const LdsOffsets& off,
                                            const u32x4 (&pb)[QB][KB][2], f32x16 (&o)[QB][DB]) {
    constexpr int VG = DB < 4 ? DB : 4;  // V^T fragments in flight per group
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rows = (kb * 32 + 16 * u) * VROW;
#pragma unroll
        for (int g = 0; g < DB; g += VG) {
          u32x4 a[VG];
#pragma unroll
          for (int i = 0; i < VG; ++i) {
            const s16x4 va = lds_read_tr16(sv + off.v[g + i] + rows);
            const s16x4 vb = lds_read_tr16(sv + off.v[g + i] + rows + 8 * VROW);
            a[i][0] = __builtin_bit_cast(u32x2, va)[0];
            a[i][1] = __builtin_bit_cast(u32x2, va)[1];
            a[i][2] = __builtin_bit_cast(u32x2, vb)[0];
            a[i][3] = __builtin_bit_cast(u32x2, vb)[1];
          }
#pragma unroll
          for (int i = 0; i < VG; ++i) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][g + i] = mfma32<BF16>(a[i], pb[qb][kb][u], o[qb][g + i]);
          }
        }
      }
    }
  }

  static __device__ __forceinline__ s16x4 lds_read_tr16(const lds_char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  }

  static __device__ __forceinline__ void run(const Params& p, lds_char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;

    // Work item (work_item); masked grids take the last query tiles (the
    // longest under a causal mask) first.
    const WorkItem item = work_item(p, blockIdx.x);
    const int bh = item.bh;
    const int qtile = MASK != kMaskNone ? (p.n_qtiles - 1 - item.step) : item.step;
    const int n = p.n;
    const int q0 = qtile * BR;
    // Query rows of this wave.  Split-KV: waves w and w+NW/2 own the same rows.
    const int qwave = SPLIT ? wave % QWAVES : wave;
    const int qw0 = q0 + qwave * QW;
    // Split-KV: the group's K/V stream and its LDS area.
    const int grp = SPLIT ? wave / QWAVES : 0;
    const int stid = SPLIT ? tid % STAGERS : tid;

    const size_t slice = (size_t)bh * (size_t)n * D;  // elements before this head
    const uint32_t slice_bytes = (uint32_t)n * D * 2;
    const auto rq = make_rsrc((const char*)p.q + slice * 2, slice_bytes);
    const auto ro = make_rsrc((char*)p.o + slice * 2, slice_bytes);
    const auto rl = make_rsrc(p.lse + (size_t)bh * n, (uint32_t)n * 4);

    // Q^T operands: for k-step s, lane holds Q[row][16s + 8*half .. +7].
    // (run_pipe starts the rest of the state from O = 0 and no keys seen.)
    State st;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + 32 * qb + (lane & 31);
#pragma unroll
      for (int s = 0; s < DK; ++s) {
        st.qf[qb][s] = __builtin_amdgcn_raw_buffer_load_b128(rq, (qrow * D + 16 * s + 8 * half) * 2, 0, 0);
        st.qf[qb][s] ^= p.q_sign;
      }
    }

    // Lane-constant LDS offsets.
    LdsOffsets off;
    {
      const int row = lane & 31;
      const int sbase = grp * STREAMB;  // this wave's K/V stream in LDS
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) off.k[ks] = sbase + row * KROW + (kslot<D>(row, 2 * ks + half) << 4);
      // V^T transposed reads: lane group g = lane/16 serves A rows (dims)
      // 16*(g%2) + lane%16 for key half g/2; as a source, lane 16g + 4e + u
      // reads key row 4*(g/2) + e at dims 16*(g%2) + 4u .. +3.  Rows 32kb+16u
      // (+8) are added as immediates; they keep key%4 and so the swizzle.
      const int g = lane >> 4;
      const int key = 4 * (g >> 1) + ((lane >> 2) & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dim = 32 * db + 16 * (g & 1) + 4 * (lane & 3);
        off.v[db] = sbase + VBASE + key * VROW + (((dim >> 3) ^ swz_v<D>(key)) << 4) + ((dim & 7) << 1);
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = stid + STAGERS * j;
        const int r = c / CPR, col = c % CPR;
        off.vst[j] = sbase + r * VROW + ((col ^ swz_v<D>(r)) << 4);
        off.kst[j] = sbase + r * KROW + (col << 4);
        // A direct-to-LDS load writes lane L's 16 bytes at the wave's base +
        // 16 L, i.e. linear slot c (row r, position col); that position of the
        // K layout holds global chunk klog(r, col), of the V layout chunk
        // col ^ swz_v(r) (an involution).
        off.gdk[j] = (r * D + klog<D>(r, col) * 8) * 2;
        off.gdv[j] = (r * D + (col ^ swz_v<D>(r)) * 8) * 2;
        // VGPR-staged loads (FA2_KV_PAD): lane chunk c in global order.
        off.gst[j] = (r * D + col * 8) * 2;
      }
      off.dma = __builtin_amdgcn_readfirstlane(sbase + (stid & ~63) * 16);
    }

    // Key tiles the workgroup's rows can see: [tfirst, tfirst + ntiles).  A
    // workgroup whose rows see no key at all still runs one fully masked tile,
    // which leaves O = 0 and LSE = +inf.
    // Key lengths apply in every mode: without a window a row's visible keys
    // are a prefix of the sequence, so a row that sees no key in the first
    // tile of a key range sees none later in it either.
    int klen = n, wl = kNoBound, wr = CAUSAL ? 0 : kNoBound, kbeg = 0;
    if (p.key_lens) klen = min(max(p.key_lens[bh / p.heads], 0), n);
    int kend = klen;
    if constexpr (CAUSAL) kend = min(klen, q0 + BR);
    if constexpr (GENERAL) {
      wl = p.wl;
      wr = p.wr;
      kbeg = max(0, q0 - wl);
      kend = min(klen, q0 + BR + wr);
    }
    const int tfirst = kbeg / BC;
    const int ntiles = kend > kbeg ? (kend + BC - 1) / BC - tfirst : 1;
    // K and V are range-checked at the keys present: rows past N, or past the
    // sequence's key length (padding, whose contents may be anything), load as
    // zeros, so a hidden key's 0 probability never meets a non-finite value.
    const uint32_t kv_bytes = (uint32_t)klen * D * 2;
    const int late = GENERAL ? max(0, qw0 + QW - 1 - wl) / BC : -1;
    const Ctx cx{rsrc_words(p.k, slice * 2, kv_bytes), rsrc_words(p.v, slice * 2, kv_bytes), ones_operand(lane),
                 ones_index(lane), lds, off, p.scale_log2, lane, tid, qw0, klen, wl, wr, late,
                 make_rsrc((const char*)p.k + slice * 2, kv_bytes), make_rsrc((const char*)p.v + slice * 2, kv_bytes)};
    if constexpr (SPLIT) {
      // Group 0 takes key tiles [tfirst, tfirst + T0) with T0 even, group 1
      // the next T0; tiles past the end are fully masked.  Both run T0
      // sub-iterations, so their barriers pair.
      const int t0 = 2 * ((ntiles + 3) / 4);
      const int first = grp == 0 ? tfirst : tfirst + t0;
      // The LDS tiles are loaded by all waves together: a rerun is the whole
      // workgroup's.
      run_pipe<!OPTIMISTIC>(cx, st, first, t0);
      if constexpr (OPTIMISTIC) {
        if (__syncthreads_or(pipe_failed(st))) run_pipe<true>(cx, st, first, t0);
      }
      merge_groups(cx, st, grp);
      if (grp != 0) return;  // group 1 handed its state to group 0
      store_output(p, st, lds, ro, rl, qw0, lane, qwave);
    } else {
      run_pipe<!OPTIMISTIC>(cx, st, tfirst, ntiles);
      if constexpr (OPTIMISTIC) {
        if (__syncthreads_or(pipe_failed(st))) run_pipe<true>(cx, st, tfirst, ntiles);
      }
      store_output(p, st, lds, ro, rl, qw0, lane, wave);
    }
  }

  // Per-wave running state.
  struct State {
    u32x4 qf[QB][DK];  // Q^T operands
    f32x16 o[QB][DB];  // O^T accumulators
    float m[QB];       // exponent base per row (base-2 domain)
    float l[QB];       // row sum (after the run: the whole sum, in every lane of the row)
    float lc[QB][2];   // checked run: row sums of queries lane%16 and 16 + lane%16
    f32x4 ls[QB];      // unchecked run: running row-sum MFMA results (see tile_sums)
    float lf[QB];      // bf16: this lane's share of the unrounded row sum (the whole sum after the run)
  };
  // bf16 rounds each probability by up to 2^-9: the output is normalised by
  // the sum of the rounded values (those the output MFMA multiplies, so one
  // dominant key gives its V row exactly), but the LSE takes the sum of the
  // unrounded ones, which is the definition.  fp16's 2^-11 keeps the LSE of
  // the rounded sum within 2^-11 (natural-log units) of it.
  static constexpr bool LSE_FP32 = BF16;
  // Pipelined schedule: first an unchecked run, rerun checked only if some row
  // overflowed (see run_pipe).  Measured: 6% faster at d = 64, 12% at d = 256,
  // 1% to 5% at d = 128.  Under the general mask d = 128 keeps only the
  // checked run: with both copies of the pipeline it does not fit the
  // registers of two waves per SIMD (it spills about 100 bytes and ran 10%
  // slower).  Under the general mask a row's window can start after the run's
  // first tile: its fixed base is taken at the first tile in which it sees a
  // key (fix_late_bases).
  static constexpr bool OPTIMISTIC = FA2_UNCHECKED_RUN && !(D == 128 && GENERAL);

  // Epilogue: O / l and LSE of one wave's rows (32 * QB), rounded and stored.
  // A lane holds 4 consecutive dims of one row per register group, so stores
  // straight from the accumulators would write 8 bytes to each of 32 rows per
  // instruction; the rows go through the wave's own LDS region instead and
  // leave as 16-byte pieces of whole rows, 64 lanes covering 1 KiB of O
  // (measured against the direct stores: +3% to +4% at d = 128 and 256, whose
  // workgroups of a round all finish together and store at once; +1% at
  // d = 64).  With the split-KV merge a wave takes the merge slot it has just
  // read (group 1 has left); otherwise every wave first passes a barrier, so
  // that no wave still reads a K/V tile.  The 16-byte chunks of a row sit at
  // chunk ^ (row mod 16) (power-of-two chunk counts; 12 chunks, d = 96:
  // plain) so that the 32 rows of a half-wave's 8-byte writes spread over the
  // banks.
  static __device__ __forceinline__ void store_output(const Params& p, const State& st, lds_char* lds,
                                                      __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rl,
                                                      int qw0, int lane, int slot) {
    constexpr int WROWS = 32 * QB;
    constexpr int WBYTES = OUT_WAVE_BYTES;
    constexpr int SWZ = (CPR & (CPR - 1)) == 0 ? (CPR < 16 ? CPR - 1 : 15) : 0;
    constexpr int MSLOT = MERGE_SLOT_BYTES;
    static_assert(!SPLIT || MSLOT % 16 == 0, "merge slots stay 16-byte aligned");
    int region;
    if constexpr (SPLIT) {
      region = slot * (MSLOT > WBYTES ? MSLOT : WBYTES);
    } else {
      __syncthreads();
      region = slot * WBYTES;
    }
    lds_char* ob = lds + region;
    const int half = lane >> 5;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = 32 * qb + (lane & 31);
      const float l_tot = st.l[qb];
      const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack2<BF16>(st.o[qb][db][4 * g + 0] * inv, st.o[qb][db][4 * g + 1] * inv);
          w[1] = pack2<BF16>(st.o[qb][db][4 * g + 2] * inv, st.o[qb][db][4 * g + 3] * inv);
          // dims 32 db + 8 g + 4 half .. +3: chunk 4 db + g, second half of it for half = 1
          *(__attribute__((address_space(3))) u32x2*)(ob + row * ROWB + (((4 * db + g) ^ (row & SWZ)) << 4) +
                                                       8 * half) = w;
        }
      }
      if (half == 0) {
        const float l_lse = LSE_FP32 ? st.lf[qb] : l_tot;
        const float lse = (l_lse > 0.f) ? (st.m[qb] + __builtin_amdgcn_logf(l_lse)) * 0.69314718055994531f
                                        : __builtin_inff();
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, (qw0 + row) * 4, 0, kStreamStore);
      }
    }
    // Whole rows out: chunk c of the wave's rows is row c / CPR, chunk c % CPR;
    // rows past N are dropped by the range-checked resource.
#pragma unroll
    for (int i = 0; i < WROWS * CPR / 64; ++i) {
      const int c = i * 64 + lane;
      const int row = c / CPR, col = c % CPR;
      const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(ob + row * ROWB + ((col ^ (row & SWZ)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, ((qw0 + row) * D + col * 8) * 2, 0, kStreamStore);
    }
  }

  // Loop-invariant context.
  struct Ctx {
    u32x4 wk, wv;  // K and V buffer descriptors as raw words (for the inline-asm loads)
    u32x4 ones;    // A operand of the row-sum MFMA (see ones_operand)
    int ones_idx;  // its sparsity index (see ones_operand)
    lds_char* lds;
    LdsOffsets off;
    float c2;
    int lane, tid, qw0;
    int n;       // keys present: N, or the sequence's key length
    int wl, wr;  // window bounds (general mask; kNoBound: none)
    int late;    // general mask: last tile in which a row of the wave can see its first key
    __amdgpu_buffer_rsrc_t rk, rv;  // K and V buffer resources for the VGPR-staged loads (FA2_KV_PAD)
    // A wave takes part in tile j if some key of it is visible to some of its rows.
    __device__ __forceinline__ bool active(int j) const {
      if constexpr (CAUSAL) return j * BC <= qw0 + QW - 1;
      if constexpr (GENERAL) return j * BC < n && j * BC <= qw0 + QW - 1 + wr && j * BC + BC - 1 >= qw0 - wl;
      return true;
    }
    // Tile j needs per-element masking (ragged tail or padding, causal
    // diagonal, window edges).
    __device__ __forceinline__ bool masked(int j) const {
      if constexpr (GENERAL)
        return (j * BC + BC > n) || (j * BC + BC - 1 > qw0 + wr) || (j * BC < qw0 + QW - 1 - wl);
      return (j * BC + BC > n) || (CAUSAL && j * BC + BC - 1 > qw0);
    }
  };

  // Register -> LDS store of V-layout chunks at a compile-time LDS offset.
  template <int BASE>
  static __device__ __forceinline__ void stage_store_v(const Ctx& cx, const u32x4 (&reg)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *(__attribute__((address_space(3))) u32x4*)(cx.lds + BASE + cx.off.vst[i]) = reg[i];
  }

  // Global -> LDS loads of one K or V tile straight into LDS buffer BASE (no
  // VGPR staging); rows past N read as zeros.  The data is in LDS once the
  // wave's vector-memory counter has drained (dma_wait).  The load is written
  // as inline asm so that the compiler, which cannot tell these LDS writes
  // from the fragment reads of other buffers, does not drain the counter
  // before every LDS read; dma_wait before each barrier is the only wait.
  static __device__ __forceinline__ void dma16(const u32x4& rsrc, const lds_char* dst, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n s_nop 0\n buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voffset), "s"(rsrc) : "memory", "m0");
  }
  template <int BASE>
  static __device__ __forceinline__ void stage_dma_k(const Ctx& cx, int tile) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) dma16(cx.wk, cx.lds + BASE + cx.off.dma + STAGERS * 16 * i, cx.off.gdk[i] + tile * GTILEB);
  }
  template <int BASE>
  static __device__ __forceinline__ void stage_dma_v(const Ctx& cx, int tile) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) dma16(cx.wv, cx.lds + BASE + cx.off.dma + STAGERS * 16 * i, cx.off.gdv[i] + tile * GTILEB);
  }
  static __device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

  // FA2_KV_PAD: one K or V tile into VGPRs (chunks in row-major order; rows
  // past the keys present read as zeros) and from there into its padded LDS
  // slot at BASE.
  static __device__ __forceinline__ void fetch_tile(const __amdgpu_buffer_rsrc_t& rsrc, const Ctx& cx, int tile,
                                                    u32x4 (&reg)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, cx.off.gst[i] + tile * GTILEB, 0, 0);
  }
  template <int BASE, bool ISV>
  static __device__ __forceinline__ void commit_tile(const Ctx& cx, const u32x4 (&reg)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *(__attribute__((address_space(3))) u32x4*)(cx.lds + BASE + (ISV ? cx.off.vst[i] : cx.off.kst[i])) = reg[i];
  }

  // ---- Pipelined schedule ------------------------------------------------
  // Iteration j issues the MFMAs of S(j+1) = K(j+1) Q^T and of
  // O^T += V(j-1)^T P(j-1)^T one at a time, each followed by its share of the
  // softmax of tile j on the VALU, so the matrix cores and the vector ALU of a
  // SIMD work side by side inside one wave.  The softmax of a tile uses the
  // current exponent base without first taking the tile's row max; a tile whose
  // probabilities could overflow (or whose base is still -inf) is caught by the
  // size of its row sums and redone through the rebase path, which takes the
  // row max, rescales O and l, and recomputes the probabilities.  The result is
  // the online softmax of the pages with a lazily moved base.  (The unchecked
  // form of run_pipe keeps the base fixed and checks once, at the end.)
  //
  // Every iteration runs the same instruction stream: a tile past the wave's
  // causal diagonal is processed as a fully masked tile (its probabilities are
  // 0), the S of the tile after the last one is computed and discarded, and
  // P(-1) is 0 against a zeroed V buffer.  Only the masking of ragged and
  // diagonal tiles and the rare rebase branch off.
  //
  // LDS: K and V each have a ring of PIPE_RING tile slots; tile t (counted
  // from the first tile of the run) lives in slot t % PIPE_RING.  The
  // sub-iterations run in groups of PIPE_G with one barrier each (pipe_group).

  static constexpr int PIPE_PF = 4;    // positions between an LDS fragment read and its first use
  static constexpr int PIPE_LEAD = 0;  // positions of softmax work before the first MFMA
  static constexpr int PIPE_TAIL = 0;  // MFMA positions after the last softmax pair
  static constexpr int PIPE_SKEW = 1;  // positions between a pair's exponentials and its packing
  static constexpr bool O_AGPR = D >= 128;  // output accumulators in AGPRs (see mfma32_acc_agpr)


  static __device__ __forceinline__ u32x4 kfrag(const lds_char* sk, const LdsOffsets& off, int kb, int ks) {
    return *(const __attribute__((address_space(3))) u32x4*)(sk + off.k[ks] + kb * 32 * KROW);
  }
  static __device__ __forceinline__ u32x4 vfrag(const lds_char* sv, const LdsOffsets& off, int kb, int u, int db) {
    const int rows = (kb * 32 + 16 * u) * VROW;
    const s16x4 va = lds_read_tr16(sv + off.v[db] + rows);
    const s16x4 vb = lds_read_tr16(sv + off.v[db] + rows + 8 * VROW);
    u32x4 a;
    a[0] = __builtin_bit_cast(u32x2, va)[0];
    a[1] = __builtin_bit_cast(u32x2, va)[1];
    a[2] = __builtin_bit_cast(u32x2, vb)[0];
    a[3] = __builtin_bit_cast(u32x2, vb)[1];
    return a;
  }

  // Keeps a value where it is computed: later code motion cannot sink the
  // instructions that produce it past this point.
  template <typename T>
  static __device__ __forceinline__ void pin(T& x) {
    asm volatile("" : "+v"(x));
  }

  // Exponentials of score registers (r0, r0+1) of block (qb, kb) against the
  // current base: exp2(c2 s - m), c2 = scale * log2(e).
  static __device__ __forceinline__ void exp_pair(const Scores& sc, const float (&m)[QB], float c2, int qb, int kb,
                                                  int r0, float& p0, float& p1) {
    p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc.s[qb][kb][r0], c2, -m[qb]));
    p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc.s[qb][kb][r0 + 1], c2, -m[qb]));
  }
  // The same pair, packed into the P operand; returns the probabilities.
  // GUARD: hidden keys give exactly 0 (also where the exponent would be NaN:
  // scale 0, or a base still at -inf).
  template <bool GUARD>
  static __device__ __forceinline__ void prob_pair(const Scores& sc, u32x4 (&pb)[QB][KB][2], const float (&m)[QB],
                                                   float c2, int qb, int kb, int r0, float& p0, float& p1) {
    exp_pair(sc, m, c2, qb, kb, r0, p0, p1);
    if constexpr (GUARD) {
      const float ninf = -__builtin_inff();
      p0 = sc.s[qb][kb][r0] == ninf ? 0.f : p0;
      p1 = sc.s[qb][kb][r0 + 1] == ninf ? 0.f : p1;
    }
    pack_pair(pb, qb, kb, r0, p0, p1);
  }
  // Round a pair of probabilities into its word of the P operand.
  static __device__ __forceinline__ void pack_pair(u32x4 (&pb)[QB][KB][2], int qb, int kb, int r0, float p0, float p1) {
    uint32_t w = pack2<BF16>(p0, p1);
    pin(w);
    pb[qb][kb][r0 >> 3][(r0 & 7) >> 1] = w;
  }

  // Softmax of a whole tile against the current base (no interleaving).
  template <bool GUARD>
  static __device__ __forceinline__ void probs_tile(const Scores& sc, u32x4 (&pb)[QB][KB][2], const float (&m)[QB],
                                                    float c2, float (&lt)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 2) {
          float p0, p1;
          prob_pair<GUARD>(sc, pb, m, c2, qb, kb, r0, p0, p1);
          la += p0;
          lb += p1;
        }
      }
      lt[qb] = la + lb;
    }
  }

  // Row sums on the matrix cores.  The packed probabilities of a 32-key tile
  // are the B operands of the output MFMA: for k-step u, lane L holds eight
  // keys of query L%32.  Both steps' words together are the 64 x 16 B operand
  // of a sparse 16x16x64 MFMA, in which the 16 values of lane L sit in
  // column L%16; lane groups 0 and 2 (L/16) hold query L%16, groups 1 and 3
  // query 16 + L%16.  The compressed A operand of lane L is row L%16; its
  // slots 0-3 meet the k of lane group 2(L/16 % 2) of B and slots 4-7 those of
  // group 2(L/16 % 2) + 1, each slot pair at the positions that the index
  // names in a group of four k.  So row i with ones in slots 0-3 (i even) or
  // 4-7 (i odd) and index positions {0,1} (i%4 < 2) or {2,3} (i%4 >= 2) sums
  // half of the values of query L%16 (i even) or 16 + L%16 (i odd), and in the
  // 16x16 result, where lane L holds rows 4(L/16)+r, registers 0 + 2 are the
  // sum of query L%16 and registers 1 + 3 that of query 16 + L%16.  These are
  // the sums of the rounded probabilities that the output MFMA consumes.
  static __device__ __forceinline__ u32x4 ones_operand(int lane) {
    const uint32_t one = BF16 ? 0x3f803f80u : 0x3c003c00u;
    return (lane & 1) ? u32x4{0u, 0u, one, one} : u32x4{one, one, 0u, 0u};
  }
  static __device__ __forceinline__ int ones_index(int lane) {
    // Two 2-bit positions per group of four k (first in the low bits), the
    // same in both 16-bit halves.
    return (lane & 2) ? (int)0xEEEEEEEEu : 0x44444444;
  }
  // Sum MFMA of query block qb of a tile, accumulated over the tile's 32-key
  // blocks (ACC: also over the tiles before it).
  template <bool ACC = false>
  static __device__ __forceinline__ void tile_sum_mfma(const Ctx& cx, const u32x4 (&pbq)[KB][2], int kb, f32x4& ct) {
    ct = smfmac16<BF16>(cx.ones, pbq[kb][0], pbq[kb][1], (kb == 0 && !ACC) ? f32x4{} : ct, cx.ones_idx);
  }
  // Sums of one tile's probabilities for every query block.
  static __device__ __forceinline__ void tile_sums(const Ctx& cx, const u32x4 (&pb)[QB][KB][2], f32x4 (&ct)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) tile_sum_mfma(cx, pb[qb], kb, ct[qb]);
    }
  }

  // Wait states after the inline-asm output MFMAs before anything the
  // compiler issues reads their accumulators (the compiler's hazard checks do
  // not see inside inline asm): 20 wait states cover the result latency of a
  // 32x32x16 MFMA, and the empty statements after them claim to modify every
  // accumulator, so that no read of O is scheduled above the wait.
  static __device__ __forceinline__ void settle_o(State& st) {
    asm volatile("s_nop 7\n s_nop 7\n s_nop 3");
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(st.o[qb][db]));
  }

  // Value of `x` held by lane `src` (every lane reads).
  static __device__ __forceinline__ float lane_value(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
  }

  // Rebase path: move each row's base to its running max, rescale O and the
  // row sums, and recompute the tile's probabilities and sums.
  static __device__ __forceinline__ void pipe_rebase(const Ctx& cx, const Scores& sc, State& st,
                                                     u32x4 (&pb)[QB][KB][2], f32x4 (&ct)[QB], float (&lt)[QB]) {
    // With O in AGPRs the output MFMAs are inline asm the compiler does not
    // track: keep the reads of O below an MFMA result latency after them.
    if constexpr (O_AGPR) settle_o(st);
    const float ninf = -__builtin_inff();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ma = ninf, mb = ninf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          ma = __builtin_fmaxf(ma, sc.s[qb][kb][r]);
          mb = __builtin_fmaxf(mb, sc.s[qb][kb][r + 1]);
        }
      }
      float mx = __builtin_fmaxf(ma, mb), lo, hi;
      halves(mx, lo, hi);
      mx = __builtin_fmaxf(lo, hi);
      const float mt = (mx == ninf) ? ninf : mx * cx.c2;
      const float m_new = __builtin_fmaxf(st.m[qb], mt);
      const float alpha = (m_new == ninf) ? 1.f : __builtin_amdgcn_exp2f(st.m[qb] - m_new);
      st.m[qb] = m_new;
      // alpha of query q lives in lanes q and q+32.
      st.lc[qb][0] *= lane_value(alpha, cx.lane & 15);
      st.lc[qb][1] *= lane_value(alpha, 16 + (cx.lane & 15));
      st.lf[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (O_AGPR) {
          // One 16-register block at a time through VGPRs: the empty asm
          // statements pin the block to its AGPRs on both sides, so the
          // compiler cannot read all of O into VGPRs at once (a peak that
          // would push loop-invariant operands out to AGPRs for the whole loop).
          asm volatile("" : "+a"(st.o[qb][db]));
          st.o[qb][db] *= alpha;
          asm volatile("" : "+a"(st.o[qb][db]));
        } else {
          st.o[qb][db] *= alpha;
        }
      }
    }
    probs_tile<true>(sc, pb, st.m, cx.c2, lt);
    tile_sums(cx, pb, ct);
  }

  // Accept the tile's sums, or send it through the rebase path.  A sum above
  // the limit (or not a number: an exponent base still at -inf) means some
  // probability may have overflowed.
  static __device__ __forceinline__ void pipe_accept(const Ctx& cx, const Scores& sc, State& st,
                                                     u32x4 (&pb)[QB][KB][2], f32x4 (&ct)[QB], float (&lt)[QB]) {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      bad |= !(ct[qb][0] + ct[qb][2] <= kTileSumLimit) || !(ct[qb][1] + ct[qb][3] <= kTileSumLimit);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0)) pipe_rebase(cx, sc, st, pb, ct, lt);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      st.lc[qb][0] += ct[qb][0] + ct[qb][2];
      st.lc[qb][1] += ct[qb][1] + ct[qb][3];
      if constexpr (LSE_FP32) st.lf[qb] += lt[qb];
    }
  }

  // The interleaved body of iteration j; S4 = (j - first) % PIPE_RING names
  // the ring slots: K(j+1) in K slot S4+1, V(j-1) in V slot S4-1 (mod the
  // ring), and the score/probability register sets alternate with j.
  template <int S4, bool CHECKED>
  static __device__ __forceinline__ void pipe_body(const Ctx& cx, State& st, Scores (&sc)[2],
                                                   u32x4 (&pb)[2][QB][KB][2], f32x4 (&ct)[QB], float (&lt)[QB]) {
    constexpr int B = S4 % 2;
    const lds_char* sk = cx.lds + ((S4 + 1) % PIPE_RING) * TILEK;                          // K(j+1)
    const lds_char* sv = cx.lds + ((S4 + PIPE_RING - 1) % PIPE_RING) * TILEV;  // V(j-1) (V ring base in off.v)
    constexpr int NMF = KB * DK * QB;               // MFMAs of each product (S and P V alike)
    constexpr int NSLOT = 2 * NMF;
    constexpr int NPAIR = QB * KB * 8;              // probability pairs of tile j
    constexpr int NKF = KB * DK, NVF = KB * 2 * DB;
    // Positions that carry softmax work: at most one probability pair each, so
    // with fewer pairs than MFMAs (d >= 128) the softmax and its row-sum MFMAs
    // finish early in the body and the sums are ready for the check at its end.
    constexpr int NVPOS = NPAIR < NSLOT - PIPE_TAIL ? NPAIR : NSLOT - PIPE_TAIL;
    static_assert(KB * 2 * DB * QB == NMF, "S and P V have equally many MFMAs");
    u32x4 kf[NKF], vf[NVF];
    float la[QB], lb[QB];
    float pe[NPAIR][2];  // exponentials waiting to be packed
    // Pairs of position ip: c in [ip * NPAIR / NVPOS, (ip + 1) * NPAIR / NVPOS).
    // Packing them (and the row-sum MFMA of each completed block of eight words).
    auto pack_position = [&](int ip) {
#pragma unroll
      for (int c = ip * NPAIR / NVPOS; c < (ip + 1) * NPAIR / NVPOS; ++c) {
        const int qb = c / (KB * 8), kb = (c / 8) % KB, r0 = 2 * (c % 8);
        pack_pair(pb[B], qb, kb, r0, pe[c][0], pe[c][1]);
        if (c % 8 == 7) tile_sum_mfma<!CHECKED>(cx, pb[B][qb], kb, ct[qb]);
      }
    };
    // Position i issues MFMA i - PIPE_LEAD (S and P V alternating), the
    // exponentials of the softmax pairs of position i and the packing of those
    // of position i - PIPE_SKEW, so that no packing waits on the latency of the
    // exponentials just issued; LDS fragments are read PIPE_PF positions before
    // their MFMA (all early ones at position 0).
#pragma unroll
    for (int i = 0; i < NSLOT + PIPE_LEAD; ++i) {
#pragma unroll
      for (int f = 0; f < NKF; ++f) {
        const int use = 2 * f * QB + PIPE_LEAD;
        if ((use - PIPE_PF > 0 ? use - PIPE_PF : 0) == i) kf[f] = kfrag(sk, cx.off, f / DK, f % DK);
      }
#pragma unroll
      for (int g = 0; g < NVF; ++g) {
        const int use = 2 * g * QB + 1 + PIPE_LEAD;
        if ((use - PIPE_PF > 0 ? use - PIPE_PF : 0) == i) vf[g] = vfrag(sv, cx.off, g / (2 * DB), (g / DB) % 2, g % DB);
      }
      const int s = i - PIPE_LEAD;
      if (s >= 0) {
        const int t = s / 2;
        if (s % 2 == 0) {
          // S MFMA t: K fragment (kb, ks), query block qb.
          const int qb = t % QB, f = t / QB, kb = f / DK, ks = f % DK;
          sc[1 - B].s[qb][kb] = mfma32<BF16>(kf[f], st.qf[qb][ks], ks == 0 ? f32x16{} : sc[1 - B].s[qb][kb]);
        } else {
          // P V MFMA t: V fragment (kb, u, db), query block qb.
          const int qb = t % QB, g = t / QB, kb = g / (2 * DB), u = (g / DB) % 2, db = g % DB;
          if constexpr (O_AGPR)
            mfma32_acc_agpr<BF16>(st.o[qb][db], vf[g], pb[1 - B][qb][kb][u]);
          else
            st.o[qb][db] = mfma32<BF16>(vf[g], pb[1 - B][qb][kb][u], st.o[qb][db]);
        }
      }
      if (i < NVPOS) {
#pragma unroll
        for (int c = i * NPAIR / NVPOS; c < (i + 1) * NPAIR / NVPOS; ++c) {
          const int qb = c / (KB * 8), kb = (c / 8) % KB, r0 = 2 * (c % 8);
          exp_pair(sc[B], st.m, cx.c2, qb, kb, r0, pe[c][0], pe[c][1]);
          if constexpr (LSE_FP32) {
            la[qb] = (kb == 0 && r0 == 0) ? pe[c][0] : la[qb] + pe[c][0];
            lb[qb] = (kb == 0 && r0 == 0) ? pe[c][1] : lb[qb] + pe[c][1];
          }
        }
      }
      if (i >= PIPE_SKEW && i - PIPE_SKEW < NVPOS) pack_position(i - PIPE_SKEW);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Positions whose packing would fall past the last MFMA position.
#pragma unroll
    for (int ip = NSLOT + PIPE_LEAD - PIPE_SKEW; ip < NVPOS; ++ip) {
      if (ip >= 0) pack_position(ip);
    }
    if constexpr (LSE_FP32) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lt[qb] = la[qb] + lb[qb];
    }
  }

  // Unchecked run under the general mask: a row that has seen no key yet
  // (base still -kUnseenBase) takes its fixed base from this tile's row max
  // if it sees a key here; its probabilities of the tiles before were 0.
  static __device__ __forceinline__ void fix_late_bases(const Ctx& cx, const Scores& sc, State& st) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc.s[qb][kb][r]);
      float lo, hi;
      halves(mx, lo, hi);
      mx = __builtin_fmaxf(lo, hi);
      if (st.m[qb] == -kUnseenBase && mx != -__builtin_inff()) st.m[qb] = mx * cx.c2;
    }
  }

  // Sub-iteration j (S4 = (j - first) % PIPE_RING): S(j+1), softmax(j), P(j-1)V(j-1).
  // Tiles past a wave's causal diagonal run as fully masked tiles (P = 0);
  // skipping them with a branch measured no faster.  CHECKED: each tile's sums
  // go through the overflow check (and the rebase path); otherwise they only
  // accumulate, and an overflow shows in the final row sums.
  template <int S4, bool CHECKED>
  static __device__ __forceinline__ void pipe_sub(const Ctx& cx, State& st, Scores (&sc)[2],
                                                  u32x4 (&pb)[2][QB][KB][2], int j) {
    constexpr int B = S4 % 2;
    if (__builtin_expect(!cx.active(j) || cx.masked(j), 0))
      mask_scores(sc[B], cx.lane, j * BC, cx.qw0, cx.n, cx.wl, cx.wr);
    if constexpr (GENERAL && !CHECKED) {
      if (__builtin_expect(j <= cx.late, 0)) fix_late_bases(cx, sc[B], st);
    }
    f32x4 ct[QB];
    float lt[QB];
    pipe_body<S4, CHECKED>(cx, st, sc, pb, CHECKED ? ct : st.ls, lt);
    if constexpr (CHECKED) {
      pipe_accept(cx, sc[B], st, pb[B], ct, lt);
    } else if constexpr (LSE_FP32) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st.lf[qb] += lt[qb];
    }
  }

  // Group of G = PIPE_RING / 2 sub-iterations j = first + r .. first + r + G-1
  // (r relative to first, H = (r / G) % 2) and one barrier.  The group reads
  // K(r+1 .. r+G) and V(r-1 .. r+G-2); at its start it sends the tiles the next
  // group reads straight to LDS: K(r+G+1 .. r+2G) and V(r+G-1 .. r+2G-2), into
  // the slots of K(r-G+1 .. r) and V(r-G-1 .. r-2), which the previous group
  // read before its barrier.  The loads have landed once every wave has drained
  // its vector-memory counter before this group's barrier.
  template <int H, int I, bool CHECKED>
  static __device__ __forceinline__ void pipe_group_subs(const Ctx& cx, State& st, Scores (&sc)[2],
                                                         u32x4 (&pb)[2][QB][KB][2], int first, int r) {
    if constexpr (I < PIPE_G) {
      pipe_sub<H * PIPE_G + I, CHECKED>(cx, st, sc, pb, first + r + I);
      pipe_group_subs<H, I + 1, CHECKED>(cx, st, sc, pb, first, r);
    }
  }
  template <int H, int I>
  static __device__ __forceinline__ void pipe_group_loads(const Ctx& cx, int first, int r) {
    if constexpr (I < PIPE_G) {
      stage_dma_k<((H * PIPE_G + PIPE_G + 1 + I) % PIPE_RING) * TILEK>(cx, first + r + PIPE_G + 1 + I);
      stage_dma_v<VBASE + ((H * PIPE_G + PIPE_G - 1 + I) % PIPE_RING) * TILEV>(cx, first + r + PIPE_G - 1 + I);
      pipe_group_loads<H, I + 1>(cx, first, r);
    }
  }
  // FA2_KV_PAD: sub-iteration I of the group first loads its share of the
  // next group's tiles (K(r+G+1+I), V(r+G-1+I)) into VGPRs and stores them to
  // their padded LDS slots after its own work.
  template <int H, int I, bool CHECKED>
  static __device__ __forceinline__ void pipe_group_subs_staged(const Ctx& cx, State& st, Scores (&sc)[2],
                                                                u32x4 (&pb)[2][QB][KB][2], int first, int r) {
    if constexpr (I < PIPE_G) {
      u32x4 kreg[CPT], vreg[CPT];
      fetch_tile(cx.rk, cx, first + r + PIPE_G + 1 + I, kreg);
      fetch_tile(cx.rv, cx, first + r + PIPE_G - 1 + I, vreg);
      pipe_sub<H * PIPE_G + I, CHECKED>(cx, st, sc, pb, first + r + I);
      commit_tile<((H * PIPE_G + PIPE_G + 1 + I) % PIPE_RING) * TILEK, false>(cx, kreg);
      commit_tile<VBASE + ((H * PIPE_G + PIPE_G - 1 + I) % PIPE_RING) * TILEV, true>(cx, vreg);
      pipe_group_subs_staged<H, I + 1, CHECKED>(cx, st, sc, pb, first, r);
    }
  }
  template <int H, bool CHECKED>
  static __device__ __forceinline__ void pipe_group(const Ctx& cx, State& st, Scores (&sc)[2],
                                                    u32x4 (&pb)[2][QB][KB][2], int first, int r) {
    if constexpr (KV_PAD) {
      pipe_group_subs_staged<H, 0, CHECKED>(cx, st, sc, pb, first, r);
    } else {
      pipe_group_loads<H, 0>(cx, first, r);
      pipe_group_subs<H, 0, CHECKED>(cx, st, sc, pb, first, r);
    }
    dma_wait();
    __syncthreads();
  }

  // Prologue loads: K(0 .. G) and V(0 .. G-2) (relative to first).
  template <int I>
  static __device__ __forceinline__ void pipe_prologue_loads(const Ctx& cx, int first) {
    if constexpr (I <= PIPE_G) {
      if constexpr (KV_PAD) {
        u32x4 reg[CPT];
        fetch_tile(cx.rk, cx, first + I, reg);
        commit_tile<I * TILEK, false>(cx, reg);
        if constexpr (I <= PIPE_G - 2) {
          fetch_tile(cx.rv, cx, first + I, reg);
          commit_tile<VBASE + I * TILEV, true>(cx, reg);
        }
      } else {
        stage_dma_k<I * TILEK>(cx, first + I);
        if constexpr (I <= PIPE_G - 2) stage_dma_v<VBASE + I * TILEV>(cx, first + I);
      }
      pipe_prologue_loads<I + 1>(cx, first);
    }
  }

  // Whether an unchecked run overflowed, or may have, in some row of this
  // lane: its row sum (of the rounded probabilities) is above the limit.
  //
  // fp16: any finite sum will do.  It means every packed probability is at
  // most 65504, so |O| stays below l * max|v| < 2^62.  bf16: a probability can
  // be as large as 2^128 (a score up to 128 base-2 units above the fixed base)
  // with the sum still finite, and then sum p v overflows the fp32
  // accumulator as soon as |v| > 2^128 / p (e.g. p = 2^121 and |v| = 300).
  // Accepting the run only while l <= 2^64 bounds every accumulator by
  // 2^64 * max|v|, finite for any |v| < 2^64; a larger sum (a score more than
  // 64 base-2 units above a row's first tile) sends the workgroup through the
  // checked run, whose probabilities are at most 2^15.
  static constexpr float kUncheckedSumLimit = BF16 ? 0x1p64f : 3.0e38f;
  static __device__ __forceinline__ bool pipe_failed(const State& st) {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bad |= !(st.l[qb] <= kUncheckedSumLimit);  // also NaN
    return bad;
  }
  // Tiles first .. first+count-1 (count >= 1) through the pipeline, in groups
  // of PIPE_G; tiles of the last group past the range are fully masked (keys
  // past N, or past the causal bound of every row).  Starts from O = 0 and
  // the row state of no keys seen.
  //
  // CHECKED = false is the optimistic form: the exponent base is fixed at the
  // row max of the first tile (a row with no visible key there gets a base so
  // low that any later visible key overflows) and no tile is checked; a
  // probability past the range of the 16-bit format makes the row sum
  // infinite (a NaN input makes it NaN), which the caller detects at the end
  // (pipe_failed) and answers by running the same tiles CHECKED, where every
  // tile's sums are checked and the base moves as needed.
  template <bool CHECKED>
  static __device__ __forceinline__ void run_pipe(const Ctx& cx, State& st, int first, int count) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      st.m[qb] = -__builtin_inff();
      st.lc[qb][0] = st.lc[qb][1] = st.lf[qb] = 0.f;
      st.ls[qb] = f32x4{};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        st.o[qb][db] = f32x16{};
        // The first reader of these zeros is an inline-asm output MFMA, for
        // which the compiler inserts no wait states after its own AGPR
        // writes: materialise them here, a whole prologue ahead, instead of
        // letting the writes sink next to that MFMA.
        if constexpr (O_AGPR) asm volatile("" : "+a"(st.o[qb][db]));
      }
    }
    Scores sc[2];
    u32x4 pb[2][QB][KB][2];
    u32x4 stg[CPT];
    // P(first-1) = 0 against a zeroed last V slot (0 * garbage could be NaN).
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) pb[1][qb][kb][0] = pb[1][qb][kb][1] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < CPT; ++i) stg[i] = u32x4{0u, 0u, 0u, 0u};
    stage_store_v<VBASE + (PIPE_RING - 1) * TILEV>(cx, stg);
    pipe_prologue_loads<0>(cx, first);
    dma_wait();
    __syncthreads();
    scores(cx.lds, cx.off, st.qf, sc[0]);  // S(first)
    __syncthreads();  // K slot 0 is rewritten by the first group's loads
    if constexpr (!CHECKED) {
      // Fixed base: the row max of the first tile (both lane halves), scaled.
      if (!cx.active(first) || cx.masked(first)) mask_scores(sc[0], cx.lane, first * BC, cx.qw0, cx.n, cx.wl, cx.wr);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc[0].s[qb][kb][r]);
        float lo, hi;
        halves(mx, lo, hi);
        mx = __builtin_fmaxf(lo, hi);
        st.m[qb] = mx == -__builtin_inff() ? -kUnseenBase : mx * cx.c2;
      }
    }
    const int count2 = (count + PIPE_G - 1) / PIPE_G * PIPE_G;
    for (int r = 0; r < count2; r += 2 * PIPE_G) {
      pipe_group<0, CHECKED>(cx, st, sc, pb, first, r);
      if (r + PIPE_G < count2) pipe_group<1, CHECKED>(cx, st, sc, pb, first, r + PIPE_G);
    }
    // P V of the last tile (relative index count2-1, V slot (count2-1) % ring,
    // probabilities in set (count2-1) % 2), an MFMA the compiler issues: an
    // MFMA result latency after the inline-asm output MFMAs it accumulates onto.
    if constexpr (O_AGPR) settle_o(st);
    if constexpr (PIPE_G % 2 == 0) {  // count2 is even: the last index is odd
      if (count2 % PIPE_RING == 0)
        pv(cx.lds + (PIPE_RING - 1) * TILEV, cx.off, pb[1], st.o);
      else
        pv(cx.lds + (PIPE_G - 1) * TILEV, cx.off, pb[1], st.o);
    } else {  // one sub-iteration per group, two slots
      static_assert(PIPE_RING == 2, "odd groups only with a 2-slot ring");
      if (count2 % 2 == 0)
        pv(cx.lds + TILEV, cx.off, pb[1], st.o);
      else
        pv(cx.lds, cx.off, pb[0], st.o);
    }
    // Each lane keeps the whole sum of its query (lane%32); with LSE_FP32 the
    // unrounded sum (the lane halves' shares added) goes to lf.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (CHECKED)
        st.l[qb] = (cx.lane & 16) ? st.lc[qb][1] : st.lc[qb][0];
      else
        st.l[qb] = (cx.lane & 16) ? st.ls[qb][1] + st.ls[qb][3] : st.ls[qb][0] + st.ls[qb][2];
      if constexpr (LSE_FP32) {
        float lo, hi;
        halves(st.lf[qb], lo, hi);
        st.lf[qb] = lo + hi;
      }
    }
  }

  // Split-KV merge: group 1 leaves (O, m, l) in LDS and group 0 combines them
  // lane by lane with the algebra of the online update.  The K/V buffers are
  // free once both groups have passed their last barrier.
  static __device__ __forceinline__ void merge_groups(const Ctx& cx, State& st, int grp) {
    typedef __attribute__((address_space(3))) float lds_float;
    __syncthreads();
    const int slot = (cx.tid % STAGERS) * MERGE_FLOATS;  // same slot for waves w and w+NW/2
    lds_float* mb = (lds_float*)cx.lds + slot;
    if (grp != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mb[(qb * DB + db) * 16 + r] = st.o[qb][db][r];
        }
        mb[QB * DB * 16 + 2 * qb] = st.m[qb];
        mb[QB * DB * 16 + 2 * qb + 1] = st.l[qb];
        mb[QB * DB * 16 + 2 * QB + qb] = st.lf[qb];
      }
    }
    __syncthreads();
    if (grp == 0) {
      const float ninf = -__builtin_inff();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m1 = mb[QB * DB * 16 + 2 * qb];
        const float l1 = mb[QB * DB * 16 + 2 * qb + 1];
        const float m0 = st.m[qb];
        const float mm = __builtin_fmaxf(m0, m1);
        const float a0 = (m0 == ninf) ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
        const float a1 = (m1 == ninf) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        st.m[qb] = mm;
        st.l[qb] = a0 * st.l[qb] + a1 * l1;
        st.lf[qb] = a0 * st.lf[qb] + a1 * mb[QB * DB * 16 + 2 * QB + qb];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) st.o[qb][db][r] = a0 * st.o[qb][db][r] + a1 * mb[(qb * DB + db) * 16 + r];
        }
      }
    }
  }

};

// The 4-wave form of d = 64 is held to 256 registers (two waves per SIMD) so
// that two of its workgroups share a CU and hide each other's prologue,
// epilogue and barrier waits; unbounded it takes 260 to 276 with bf16 or the
// general mask, one wave per SIMD.  The other forms fill a CU with one
// workgroup (8 waves, or LDS- and register-bound d = 96 and 256).
template <int D, int BC, int NW, int QB, int KVG, bool BF16, int MASK>
__global__ void __launch_bounds__(NW * 64)
    __attribute__((amdgpu_waves_per_eu((FA2_W4_TWO_PER_SIMD && NW == 4 && (D == 64 || (D == 128 && QB == 1))) ? 2 : 1)))
    fa2_fwd_kernel(const Params p) {
  extern __shared__ __attribute__((aligned(16))) char lds_generic[];
  Fa2Fwd<D, BC, NW, QB, KVG, BF16, MASK>::run(
      p, (__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)lds_generic);
}

}  // namespace fa2
