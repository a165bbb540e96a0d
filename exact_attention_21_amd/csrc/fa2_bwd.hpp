// FlashAttention-2 backward kernels for gfx950 (CDNA4), wave64 MFMA.
//
// What they compute (per batch b, head h), given the forward's O and LSE and
// the output gradient dO, with S = scale * Q K^T over the keys each query
// sees (all, j <= i under the causal mask, or the forward's general mask: a
// sliding window below a per-sequence key length) and P = exp(S - LSE) (the
// forward's probabilities, recomputed; 0 for hidden keys):
//   dV = P^T dO
//   dP = dO V^T,   Delta_i = sum_d dO[i,d] O[i,d],   dS = P * (dP - Delta)
//   dQ = scale * dS K,   dK = scale * dS^T Q
// Method: "第 15 章 FA2 前向：Tiling 与 Online Softmax" (yangyitao.com), the
// chapter's closing paragraph on the backward: S and P are recomputed from Q,
// K and the stored LSE instead of being read, and the loop runs over key
// tiles outside and query tiles inside; the arithmetic is the chain rule
// through the softmax of the forward's definition ("FlashAttention-2 MMA
// 代码学习" (chuoer47.github.io), step 0).
//
// gfx950 design (where it departs from the pages' outline):
//   * The pages accumulate dQ with atomic adds from every key tile.  Here two
//     kernels share the work without atomics, and the results do not depend
//     on the order in which workgroups run:
//       - Fa2BwdQ (query rows stationary, key tiles streamed): Delta and the
//         base-2 LSE of its rows (written to a workspace, negated), then
//         S^T, dP^T, dS^T and dQ^T += K^T dS^T.  Launched first.
//       - Fa2BwdKV (key rows stationary, query tiles streamed, the pages'
//         loop order): S, dP, dS, dV^T += dO^T P and dK^T += Q^T dS.
//     S and dP are computed in both, 7 matrix products in all instead of 5.
//   * Every product is v_mfma_f32_32x32x16_{f16,bf16} with fp32 accumulation.
//     The operand that stays in registers (Q^T and dO^T in Fa2BwdQ, K^T and
//     V^T in Fa2BwdKV) is the B operand of the score products, so the score
//     accumulators hold one row (or key) per lane and 16 keys (or queries)
//     in registers; registers 8u..8u+7 of such an accumulator are, packed to
//     16 bits, the B operand of the gradient product for k-step u, exactly as
//     the forward feeds P to its output product.  The A operands of the
//     gradient products (K^T, dO^T, Q^T) are read from LDS transposed, with
//     ds_read_b64_tr_b16.
//   * Streamed tiles go from global memory straight into a 2-slot LDS ring
//     (buffer_load ... lds), one barrier per tile.  A streamed tile is read
//     both as plain rows and transposed; its 16-byte chunks are permuted
//     per row (bwd_pos) so that both reads are free of LDS bank conflicts.
//   * The dP accumulators start at -Delta instead of 0, so the product gives
//     dP - Delta and dS = P (dP - Delta) is one multiply per element.
//   * Tiles that hold a hidden (row, key) pair run their own instantiation
//     of the tile body, with the per-element mask; they are a prefix and a
//     suffix of each workgroup's tile range (window edges, causal diagonal,
//     key length, ragged N), the tiles between carry no mask arithmetic.
//   * Each wave runs a software pipeline: step j issues the MFMAs of the next
//     block's score products and of the previous block's gradient products
//     one at a time, each followed by a share of block j's exponentials, dS
//     and packing.
//   * Rows past N load as zeros from range-checked buffer resources and
//     contribute exactly zero; out-of-range stores are dropped by the same
//     check.
//
// Precision: S, dP, Delta and the gradient accumulators are fp32; P and dS
// are rounded (to nearest even) to the input dtype before the products that
// take them, as the forward rounds P; the gradients are rounded to the input
// dtype once, at the end.
#pragma once

#include "fa2_kernel.hpp"

#include <type_traits>

namespace fa2 {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // natural-log LSE of the forward, [B*H, N]
  float* delta;      // workspace [2, B*H, N]: -Delta, then -LSE * log2(e) (Fa2BwdQ writes, Fa2BwdKV reads)
  void* dq;
  void* dk;
  void* dv;
  int n;        // sequence length N
  int bh;       // B * H
  int n_tiles;      // stationary tiles per (batch*head) slice of the kernel launched
  int group;        // slices per group of the work order (bwd_work_item)
  int phase_tiles;  // steps per phase of the work order (bwd_work_item; n_tiles: one phase)
  float scale;  // softmax scale (any finite value)
  float c2;     // scale * log2(e): scores to the base-2 exponent domain
  // General mask (the forward's): key j is visible to query i iff
  // j < key_len(b), j >= i - wl and j <= i + wr (kNoBound: no bound).
  int wl;
  int wr;
  const int* key_lens;  // B lengths (clamped to [0, N]) or null
  int heads;            // H, to find the batch of a (batch*head) slice
};

constexpr float kLog2e = 1.4426950408889634f;


// Work item of workgroup wg: its (batch*head) slice and its step (tile
// index, counted from the longest tile under a mask).  The steps are taken in
// phases of p.phase_tiles (the last may be shorter), every step of a phase
// before the next phase; inside a phase the slices are taken in groups of
// p.group, every step of a group before the next group, the step varying
// slowest inside a group: with a group of (a multiple of) 8 slices each XCD
// (workgroups are dealt to the 8 XCDs round robin) runs the tiles of the same
// few slices together, so the tiles they stream (K and V, or Q and dO) are
// read from its L2 instead of HBM (the forward's order, work_item).  Two
// phases put the long steps of every group before the short ones, so that
// the last groups' long tiles do not start at the end of the launch.
struct BwdItem {
  int bh;
  int step;
};
__device__ __forceinline__ BwdItem bwd_work_item(const BwdParams& p, int wg) {
  const int phase = wg / (p.bh * p.phase_tiles);
  const int step0 = phase * p.phase_tiles;
  wg -= step0 * p.bh;
  const int steps = min(p.phase_tiles, p.n_tiles - step0);
  const int span = p.group * steps;
  const int g = wg / span;
  const int r = wg - g * span;
  const int size = min(p.group, p.bh - g * p.group);
  const int step = r / size;
  return {g * p.group + (r - step * size), step0 + step};
}

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1 in order: the
// pipelines below index their register arrays with these compile-time
// values, which does not depend on the loop unroller's size limits (a loop
// it left rolled would put the arrays in scratch memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Position of 16-byte chunk c of row r of a streamed tile (bwd_pos), and the
// chunk held at position p (bwd_chunk, its inverse).  A tile is read two ways:
//  * plain: 16 lanes read 16 consecutive rows at one chunk, so the 16 chunks
//    must fall in distinct 16-byte bank groups of the 256-byte LDS line;
//  * transposed (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows 4a+e
//    (e = 0..3) at one aligned group of 4 chunks, so those 16 chunks must too.
// d = 32 (4 chunks, four rows per line, the line quarter given by r%4): the
// XOR follows r/4 % 4, so the four rows of 16 that share a line quarter take
// four different chunk positions; a transposed read covers whole rows, one
// per line quarter.  d = 64 (8 chunks, two rows per line, the line half given
// by r%2): bits 0-1 of the XOR walk the four aligned 4-row groups of 16 rows
// and bit 2 follows r/2 % 2, which puts rows 4a and 4a+2 (same line half) in
// different 4-chunk halves.  d = 128 and 256 (16 or 32 chunks, whole lines):
// bits 2-3 follow r%4 (the four rows of a transposed read in four different
// 4-chunk groups) and bits 0-1 follow r/4 % 4, so 16 consecutive rows take 16
// distinct values.  d = 96 (12 chunks, rows starting at bank groups 12r mod
// 16, which repeat every 4 rows): the chunks rotate by r/4 % 4 within the
// row, which separates rows 4 apart for the plain read; the four rows of a
// transposed read already start 12 groups apart.  (Every rule was checked
// exhaustively for both reads.)  All depend on r only through r%16.
template <int D>
constexpr int bwd_pos(int row, int c) {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "backward head dims");
  if constexpr (D == 32) return c ^ ((row >> 2) & 3);
  if constexpr (D == 64) return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  if constexpr (D == 96) return (c + ((row >> 2) & 3)) % 12;
  return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
}
template <int D>
constexpr int bwd_chunk(int row, int p) {
  if constexpr (D == 96) return (p + 12 - ((row >> 2) & 3)) % 12;
  return bwd_pos<D>(row, p);  // the XOR rules are involutions
}

template <int D, bool BF16>
struct BwdBase {
  static constexpr int ROWB = D * 2;  // bytes per row
  static constexpr int CPR = D / 8;   // 16-byte chunks per row
  static constexpr int DK = D / 16;   // 16-deep k-steps over the head dim
  static constexpr int DB = D / 32;   // 32-dim blocks of a gradient accumulator
  typedef __attribute__((address_space(3))) char lds_char;

  static __device__ __forceinline__ u32x4 lds16(const lds_char* p) {
    return *(const __attribute__((address_space(3))) u32x4*)p;
  }
  static __device__ __forceinline__ f32x4 lds_f4(const lds_char* p) {
    return *(const __attribute__((address_space(3))) f32x4*)p;
  }
  static __device__ __forceinline__ s16x4 tr16(const lds_char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  }

  // Plain read: lane L reads row L%32 at chunk 2ks + L/32 (dims 16ks + 8(L/32)
  // .. +7): the A operand [32 rows x 16 dims] of a score product.  Rows of
  // later 32-row blocks are added as immediates (multiples of 16 rows keep
  // the swizzle).
  static constexpr int plain_off(int lane, int ks) {
    const int row = lane & 31;
    return row * ROWB + (bwd_pos<D>(row, 2 * ks + (lane >> 5)) << 4);
  }
  // Transposed read of dims 32db.. of 16 rows: lane group g = L/16 serves A
  // rows (dims) 16(g%2) + L%16; as a source, lane 16g + 4e + u reads row
  // 4(g/2) + e (+8 for the second read) at dims 32db + 16(g%2) + 4u .. +3.
  // The two reads give the A operand [32 dims x 16 rows] with its k index
  // ordered rows {4h + e, 8 + 4h + e} for lane half h, the order of
  // registers 8u..8u+7 of a score accumulator.
  static constexpr int tr_off(int lane, int db, int second) {
    const int g = lane >> 4;
    const int row = 4 * (g >> 1) + ((lane >> 2) & 3) + 8 * second;
    const int c = 4 * db + 2 * (g & 1) + ((lane & 3) >> 1);
    return row * ROWB + (bwd_pos<D>(row, c) << 4) + 8 * (lane & 1);
  }
  static __device__ __forceinline__ u32x4 tr_frag(const lds_char* p0, const lds_char* p1) {
    const s16x4 a = tr16(p0);
    const s16x4 b = tr16(p1);
    u32x4 r;
    r[0] = __builtin_bit_cast(u32x2, a)[0];
    r[1] = __builtin_bit_cast(u32x2, a)[1];
    r[2] = __builtin_bit_cast(u32x2, b)[0];
    r[3] = __builtin_bit_cast(u32x2, b)[1];
    return r;
  }

  // x ^ k, issued where it is used: the asm keeps the compiler from holding
  // one register per constant k through the loop (it would hoist the XORs of
  // a loop-invariant x) or from merging equal ones.
  static __device__ __forceinline__ int xor_at(int x, int k) {
    if (k == 0) return x;
    int r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(k), "v"(x));
    return r;
  }

  // LDS pointer of a byte address.
  static __device__ __forceinline__ const lds_char* at(int addr) { return (const lds_char*)(uintptr_t)(uint32_t)addr; }
  // LDS byte address of a pointer.
  static __device__ __forceinline__ int addr_of(const lds_char* p) { return (int)(uint32_t)(uintptr_t)p; }

  // Addresses of the fragment reads of a tile at LDS byte address `base`, a
  // multiple of ROWB (the slots sit at multiples of ROWB from the start of
  // the kernels' dynamic LDS, address 0: they declare no static LDS).
  // Under the XOR chunk permutations (every head dim but 96) chunk c of a row
  // sits at byte 16 (c ^ f) = 16 c ^ 16 f of it, below ROWB (a power of
  // two), so the plain read of k-step ks is plain_off(lane, 0) ^ 32 ks and
  // the transposed read of dims 32 db.. is tr_off(lane, 0, s) ^ 64 db, each
  // plus the base.  XOR_ = true: three lane offsets and one XOR at each
  // read, for the d = 256 dK/dV kernel, which spilled with one register per
  // read offset held through the loop (and each spill reload waited for the
  // tile loads in flight).  XOR_ = false: one offset per read, for the
  // kernels that fit their registers, where the XORs only cost issue slots
  // (measured 2.5% to 5% slower at d <= 128, 4% to 5% in the d = 256 dQ
  // kernel).
  // The XOR forms, for every lane (checked at compile time where used).
  static constexpr bool xor_forms_hold() {
    for (int lane = 0; lane < 64; ++lane) {
      for (int ks = 0; ks < DK; ++ks)
        if (plain_off(lane, ks) != (plain_off(lane, 0) ^ (32 * ks))) return false;
      for (int db = 0; db < DB; ++db)
        for (int s = 0; s < 2; ++s)
          if (tr_off(lane, db, s) != (tr_off(lane, 0, s) ^ (64 * db))) return false;
    }
    return 32 * (DK - 1) < ROWB && 64 * (DB - 1) < ROWB;
  }
  template <bool XOR_>
  struct FragOffT {
    static constexpr bool XOR = XOR_ && D != 96;
    static_assert(!XOR || xor_forms_hold(), "fragment offsets are a lane base XOR a constant");
    int p0, t0, t1;
    int pk[XOR ? 1 : DK], tk[XOR ? 1 : DB][2];
    __device__ __forceinline__ explicit FragOffT(int lane) {
      p0 = plain_off(lane, 0);
      t0 = tr_off(lane, 0, 0);
      t1 = tr_off(lane, 0, 1);
      if constexpr (!XOR) {
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) pk[ks] = plain_off(lane, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          tk[db][0] = tr_off(lane, db, 0);
          tk[db][1] = tr_off(lane, db, 1);
        }
      }
    }
    __device__ __forceinline__ int plain(int base, int ks) const {
      if constexpr (XOR) return xor_at(p0 + base, 32 * ks);
      return pk[ks] + base;
    }
    __device__ __forceinline__ int tr(int base, int db, int second) const {
      if constexpr (XOR) return xor_at((second ? t1 : t0) + base, 64 * db);
      return tk[db][second] + base;
    }
  };

  // Global -> LDS copies that bypass the VGPRs: lane L of the wave writes its
  // 16 (or 4) bytes at the LDS address `dst` + 16 L (4 L).  Written as inline
  // asm so that the compiler does not drain the memory counter before every
  // LDS read; dma_wait before each barrier is the only wait.
  static __device__ __forceinline__ void dma16(const u32x4& rsrc, const lds_char* dst, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n s_nop 0\n buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voffset), "s"(rsrc) : "memory", "m0");
  }
  static __device__ __forceinline__ void dma4(const u32x4& rsrc, const lds_char* dst, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n s_nop 0\n buffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voffset), "s"(rsrc) : "memory", "m0");
  }
  static __device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

  // Staging of a ROWS-row tile by T threads: thread t copies linear LDS slots
  // t + T j; slot s is row s / CPR at position s % CPR, which holds chunk
  // bwd_chunk(row, s % CPR) of that row.  PERIODIC (T a multiple of CPR):
  // slot j of a thread is RJ = T / CPR rows below slot 0, and as the chunk
  // permutations depend on the row only through r % 16, the offsets repeat
  // every PER = 16 / gcd(16, RJ) slots up to whole rows: PER lane offsets,
  // each made opaque at every staging so that the compiler adds the row
  // terms there instead of holding one register per slot (used at d = 256,
  // where those registers spilled).  Otherwise one offset per slot.
  template <int ROWS, int T, bool PERIODIC>
  struct Stager {
    static constexpr int CPT = ROWS * CPR / T;
    static_assert(CPT >= 1 && (ROWS * CPR) % T == 0, "staging split");
    static constexpr int RJ = PERIODIC && T % CPR == 0 ? T / CPR : 0;
    static constexpr int PER0 = RJ == 0 ? CPT : RJ % 16 == 0 ? 1 : RJ % 8 == 0 ? 2 : RJ % 4 == 0 ? 4 : RJ % 2 == 0 ? 8 : 16;
    static constexpr int PER = PER0 < CPT ? PER0 : CPT;
    int goff[PER];  // global byte offset within the tile of slots 0 .. PER-1
    int lds0;       // this wave's first slot (bytes)
    static constexpr int slot_off(int tid, int j) {
      const int s = tid + T * j;
      const int row = s / CPR;
      return (row * D + bwd_chunk<D>(row, s % CPR) * 8) * 2;
    }
    // The period, for every thread (checked at compile time).
    static constexpr bool period_holds() {
      for (int tid = 0; tid < T; ++tid)
        for (int j = 0; j < CPT; ++j)
          if (slot_off(tid, j) != slot_off(tid, j % PER) + (j - j % PER) * RJ * ROWB) return false;
      return true;
    }
    static_assert(RJ == 0 || period_holds(), "staging offsets repeat every PER slots up to whole rows");
    __device__ __forceinline__ Stager(int tid) {
#pragma unroll
      for (int j = 0; j < PER; ++j) goff[j] = slot_off(tid, j);
      lds0 = (tid & ~63) * 16;
    }
    // Tile of rows r0.. into LDS at dst.  The row term stays in the VGPR
    // offset: the range check that zero-fills rows past the end covers it.
    __device__ __forceinline__ void stage(const u32x4& rsrc, const lds_char* dst, int r0) const {
      int g[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        g[i] = goff[i];
        if constexpr (RJ != 0) asm volatile("" : "+v"(g[i]));
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j)
        dma16(rsrc, dst + lds0 + T * 16 * j, g[j % PER] + (r0 + (j - j % PER) * RJ) * ROWB);
    }
  };

  // Gradient accumulators in AGPRs (AGPR = true: wide head dims, one wave per
  // SIMD, the arch VGPRs hold the rest) go through the forward's inline-asm
  // MFMA, under its rules: A and B are never written by VALU just before it
  // (the B operands are packed a step earlier), the two MFMAs of one
  // accumulator in a step are other MFMAs apart, and compiler-issued reads
  // of the accumulators come only after settle().
  template <bool AGPR>
  static __device__ __forceinline__ void acc_zero(f32x16 (&x)[DB]) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      x[db] = f32x16{};
      if constexpr (AGPR) asm volatile("" : "+a"(x[db]));
    }
  }
  template <bool AGPR>
  static __device__ __forceinline__ void acc_mfma(f32x16& c, const u32x4& a, const u32x4& b) {
    if constexpr (AGPR)
      mfma32_acc_agpr<BF16>(c, a, b);
    else
      c = mfma32<BF16>(a, b, c);
  }
  // Wait states between the last inline-asm MFMA of an accumulator and a
  // compiler-issued read of it (a 32x32 MFMA's result is readable 18 passes
  // after issue); the pins keep the reads behind the wait.
  template <bool AGPR>
  static __device__ __forceinline__ void settle(f32x16 (&x)[DB]) {
    if constexpr (AGPR) {
      asm volatile("s_nop 7\n s_nop 7\n s_nop 3");
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(x[db]));
    }
  }

  // Registers 8u..8u+7 of a score accumulator, rounded and packed: the B
  // operand of a gradient product for k-step u.
  static __device__ __forceinline__ void pack_operand(const float (&x)[16], u32x4 (&b)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int m = 0; m < 4; ++m) b[u][m] = pack2<BF16>(x[8 * u + 2 * m], x[8 * u + 2 * m + 1]);
    }
  }

  // A gradient accumulator [32 dims x 32 rows] times `mul`, rounded and
  // stored: lane L holds row `row` (its column) and, in register group g,
  // dims 32db + 8g + 4(L/32) .. +3, stored as 8 bytes.
  static __device__ __forceinline__ void store_grad(__amdgpu_buffer_rsrc_t r, const f32x16 (&acc)[DB], int row,
                                                    int lane, float mul) {
    const int h = lane >> 5;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack2<BF16>(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul);
        w[1] = pack2<BF16>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
        __builtin_amdgcn_raw_buffer_store_b64(w, r, (row * D + 32 * db + 8 * g + 4 * h) * 2, 0, 0);
      }
    }
  }
};

// ---- dQ (and Delta): query rows stationary, key tiles streamed ----------
template <int D, int NW, bool BF16, int MASK>
struct Fa2BwdQ : BwdBase<D, BF16> {
  static constexpr bool CAUSAL = MASK == kMaskCausal;
  static constexpr bool GENERAL = MASK == kMaskGeneral;
  using Base = BwdBase<D, BF16>;
  using Base::CPR;
  using Base::DB;
  using Base::DK;
  using Base::ROWB;
  using typename Base::lds_char;
  static constexpr int THREADS = NW * 64;
  static constexpr int BQ = NW * 32;  // query rows per workgroup (32 per wave)
  // Keys per streamed tile: 128 at d = 32 and 64, 64 at d = 128 (two tiles in
  // LDS, 64 KiB, so that two workgroups share a CU) and 256 (128 KiB).
  static constexpr int BC = D <= 64 ? 128 : 64;
  // dQ accumulators in AGPRs at d = 256 (one wave per SIMD).
  static constexpr bool ACC_AGPR = D >= 256;
  static constexpr int KB = BC / 32;
  static constexpr int TILEB = BC * ROWB;
  static constexpr int SLOTB = 2 * TILEB;  // one K tile and one V tile
  static constexpr int LDS_BYTES = 2 * SLOTB;
  // Fragment and staging addresses (FragOffT, Stager): one register per
  // fragment read (the XOR at each read measured 4% to 5% slower at d = 256,
  // where this kernel does not spill either way); staging offsets kept to the
  // permutation's period at d = 256.
  static constexpr bool XOR_ADDR = false;
  static constexpr bool PERIODIC_STAGE = D >= 256;
  using FragOff = typename Base::template FragOffT<XOR_ADDR>;
  using St = typename Base::template Stager<BC, THREADS, PERIODIC_STAGE>;
  static_assert(!FragOff::XOR || SLOTB % ROWB == 0, "slot bases keep the fragment offsets' XOR bits");
  // Software pipeline over the KB 32-key blocks of a tile: step j issues the
  // MFMAs of S(j+1) and dP(j+1) (NSD, S and dP alternating) and of
  // dQ += K^T dS(j-1) (NQ), one at a time, each followed by its share of the
  // VALU work of block j (8 pairs of probabilities: exponential, dS, packing).
  static constexpr int NSD = 2 * DK;
  static constexpr int NQ = 2 * DB;
  static constexpr int NPOS = NSD + NQ;
  static constexpr int PF = 3;  // positions between a fragment's LDS read and its MFMA

  static __device__ __forceinline__ void run(const BwdParams& p, lds_char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const BwdItem item = bwd_work_item(p, blockIdx.x);
    const int step = item.step;
    const int bh = item.bh;
    // Under a mask the last query tiles (causal: the most keys) first.
    const int qtile = MASK != kMaskNone ? p.n_tiles - 1 - step : step;
    const int n = p.n;
    const int q0 = qtile * BQ;
    const int qw0 = q0 + 32 * wave;
    const int myq = qw0 + (lane & 31);

    const size_t slice = (size_t)bh * (size_t)n * D;
    const uint32_t bytes = (uint32_t)n * D * 2;
    const auto rq = make_rsrc((const char*)p.q + slice * 2, bytes);
    const auto rdo = make_rsrc((const char*)p.dout + slice * 2, bytes);
    const auto ro = make_rsrc((const char*)p.o + slice * 2, bytes);
    const auto rdq = make_rsrc((char*)p.dq + slice * 2, bytes);
    const auto rl = make_rsrc(p.lse + (size_t)bh * n, (uint32_t)n * 4);
    // Workspace: -Delta of every row, then -LSE * log2(e) of every row.
    const auto rnd = make_rsrc(p.delta + (size_t)bh * n, (uint32_t)n * 4);
    const auto rnl = make_rsrc(p.delta + ((size_t)p.bh + bh) * n, (uint32_t)n * 4);

    // Q^T and dO^T operands (lane: row myq, dims 16ks + 8h .. +7), and Delta
    // of the row from dO and O as stored.
    u32x4 qf[DK], df[DK];
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      const int off = (myq * D + 16 * ks + 8 * h) * 2;
      qf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      df[ks] = __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0);
      const u32x4 of = __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0);
      if constexpr (BF16) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, df[ks]), b = __builtin_bit_cast(bf16x8, of);
#pragma unroll
        for (int i = 0; i < 8; ++i) dsum = __builtin_fmaf((float)a[i], (float)b[i], dsum);
      } else {
        const f16x8 a = __builtin_bit_cast(f16x8, df[ks]), b = __builtin_bit_cast(f16x8, of);
#pragma unroll
        for (int i = 0; i < 8; ++i) dsum = __builtin_fmaf((float)a[i], (float)b[i], dsum);
      }
    }
    float lo, hi;
    halves(dsum, lo, hi);
    const float ndelta = -(lo + hi);
    const float nl2 = -__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, myq * 4, 0, 0)) * kLog2e;
    if (h == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ndelta), rnd, myq * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nl2), rnl, myq * 4, 0, 0);
    }
    // dP^T accumulators start at -Delta, so the product gives dP - Delta.
    f32x16 dp0;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp0[r] = ndelta;

    // Lane-constant LDS offsets.
    const FragOff fo(lane);
    const St st(tid);
    // K and V are range-checked at the keys present (N, or the sequence's
    // key length: rows past it may hold anything and are never read).
    int klen = n, wl = kNoBound, wr = kNoBound;
    if constexpr (GENERAL) {
      if (p.key_lens) klen = min(max(p.key_lens[bh / p.heads], 0), n);
      wl = p.wl;
      wr = p.wr;
    }
    const u32x4 wk = rsrc_words(p.k, slice * 2, (uint32_t)klen * D * 2);
    const u32x4 wv = rsrc_words(p.v, slice * 2, (uint32_t)klen * D * 2);

    f32x16 dq[DB];
    Base::template acc_zero<ACC_AGPR>(dq);

    // Key tiles that some row of the workgroup sees: [tfirst, tend).  A tile
    // takes the per-element mask when it holds a key past N (or the key
    // length) or a key some row of the workgroup does not see.
    int kbeg = 0, kend = n;
    if constexpr (CAUSAL) kend = min(n, q0 + BQ);
    if constexpr (GENERAL) {
      kbeg = max(0, q0 - wl);
      kend = min(klen, q0 + BQ + wr);  // q0 + BQ - 1 + wr + 1
    }
    const int tfirst = kbeg / BC;
    const int tend = kend > kbeg ? (kend + BC - 1) / BC : tfirst;
    // The masked tiles are a prefix [tfirst, m1) (keys before the last row's
    // left bound) and a suffix [m2, tend) (keys past the key length, or
    // after the first row's right bound; causal: after the first row).
    const int lb = q0 + BQ - 1 - wl;  // tiles starting before this key are masked
    const int m1 = min(tend, max(tfirst, GENERAL && lb > 0 ? (lb + BC - 1) / BC : tfirst));
    int rcut = klen / BC;  // first tile holding a key at or past the key length
    if constexpr (CAUSAL) rcut = min(rcut, (q0 + 1) / BC);
    if constexpr (GENERAL) rcut = min(rcut, (int)(((int64_t)q0 + wr + 1) / BC));
    const int m2 = min(tend, max(m1, rcut));
    auto tile = [&](int t, auto masked_c) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_c)::value;
      Base::dma_wait();
      __syncthreads();
      const int slot = Base::addr_of(lds) + ((t - tfirst) & 1) * SLOTB;
      if (t + 1 < tend) {
        const lds_char* nk = lds + ((t + 1 - tfirst) & 1) * SLOTB;
        st.stage(wk, nk, (t + 1) * BC);
        st.stage(wv, nk + TILEB, (t + 1) * BC);
      }
      const int k0 = t * BC;
      f32x16 sc[2], dp[2];  // S^T and dP^T - Delta of blocks of either parity
      u32x4 b[2][2];        // packed dS^T of blocks of either parity
      // A operand of MFMA `pos` of the step that works on block j: S(j+1)
      // and dP(j+1) (K and V rows), then dQ(j-1) (K^T, transposed read).
      auto frag = [&](int j, int pos) __attribute__((always_inline)) -> u32x4 {
        if (pos < NSD) {
          const int kb = j + 1, ks = pos / 2;
          return Base::lds16(Base::at(fo.plain(slot, ks)) + (pos % 2 ? TILEB : 0) + kb * 32 * ROWB);
        }
        const int kb = j - 1, u = (pos - NSD) / DB, db = (pos - NSD) % DB;
        const int rows = (kb * 32 + 16 * u) * ROWB;
        return Base::tr_frag(Base::at(fo.tr(slot, db, 0)) + rows, Base::at(fo.tr(slot, db, 1)) + rows);
      };
      auto active = [&](int j, int pos) __attribute__((always_inline)) { return pos < NSD ? j + 1 < KB : j >= 1; };
      auto issue = [&](int j, int pos, const u32x4& a) __attribute__((always_inline)) {
        if (pos < NSD) {
          const int kb = j + 1, ks = pos / 2;
          if (pos % 2 == 0)
            sc[kb % 2] = mfma32<BF16>(a, qf[ks], ks == 0 ? f32x16{} : sc[kb % 2]);
          else
            dp[kb % 2] = mfma32<BF16>(a, df[ks], ks == 0 ? dp0 : dp[kb % 2]);
        } else {
          const int kb = j - 1, u = (pos - NSD) / DB, db = (pos - NSD) % DB;
          Base::template acc_mfma<ACC_AGPR>(dq[db], a, b[kb % 2][u]);
        }
      };
      // VALU work of pair c of block j: registers 2c, 2c+1 (keys
      // kr0 + 8(r/4) + 4h + r%4 of row myq).
      auto pair = [&](int j, int c) __attribute__((always_inline)) {
        float x[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * c + e;
          x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j % 2][r], p.c2, nl2));
          if constexpr (MASKED) {
            const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool hide = GENERAL ? (key >= klen || key > myq + wr || key < myq - wl)
                                      : (key >= n || (CAUSAL && key > myq));
            if (hide) x[e] = 0.f;
          }
          x[e] *= dp[j % 2][r];
        }
        b[j % 2][c / 4][c % 4] = pack2<BF16>(x[0], x[1]);
      };
      // Prologue: S(0) and dP(0).
      static_for<0, NSD>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pos = decltype(pc)::value;
        const u32x4 a = frag(-1, pos);
        issue(-1, pos, a);
      });
      static_for<0, KB>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        u32x4 fr[NPOS];
        static_for<0, (PF < NPOS ? PF : NPOS)>([&](auto pc) __attribute__((always_inline)) {
          constexpr int pos = decltype(pc)::value;
          if (active(j, pos)) fr[pos] = frag(j, pos);
        });
        static_for<0, NPOS>([&](auto pc) __attribute__((always_inline)) {
          constexpr int pos = decltype(pc)::value;
          if constexpr (pos + PF < NPOS) {
            if (active(j, pos + PF)) fr[pos + PF] = frag(j, pos + PF);
          }
          if (active(j, pos)) issue(j, pos, fr[pos]);
          static_for<pos * 8 / NPOS, (pos + 1) * 8 / NPOS>(
              [&](auto cc) __attribute__((always_inline)) { pair(j, decltype(cc)::value); });
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      // Epilogue: dQ(KB-1).
      static_for<NSD, NPOS>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pos = decltype(pc)::value;
        const u32x4 a = frag(KB, pos);
        issue(KB, pos, a);
      });
    };
    if (tend > tfirst) {
      st.stage(wk, lds, tfirst * BC);
      st.stage(wv, lds + TILEB, tfirst * BC);
    }
    int t = tfirst;
    if constexpr (GENERAL) {
      for (; t < m1; ++t) tile(t, std::true_type{});
    }
    for (; t < m2; ++t) tile(t, std::false_type{});
    for (; t < tend; ++t) tile(t, std::true_type{});
    Base::template settle<ACC_AGPR>(dq);
    Base::store_grad(rdq, dq, myq, lane, p.scale);
  }
};

// ---- dK and dV: key rows stationary, query tiles streamed -----------------
template <int D, int NW, bool BF16, int MASK>
struct Fa2BwdKV : BwdBase<D, BF16> {
  static constexpr bool CAUSAL = MASK == kMaskCausal;
  static constexpr bool GENERAL = MASK == kMaskGeneral;
  using Base = BwdBase<D, BF16>;
  using Base::CPR;
  using Base::DB;
  using Base::DK;
  using Base::ROWB;
  using typename Base::lds_char;
  static constexpr int THREADS = NW * 64;
  static constexpr int BK = NW * 32;  // key rows per workgroup (32 per wave)
  static constexpr int BQ = D >= 256 ? 64 : 128;  // query rows per streamed tile (LDS: two slots)
  static constexpr int QBLK = BQ / 32;
  static constexpr int TILEB = BQ * ROWB;
  // Slot: Q tile, dO tile, then -LSE * log2(e) and -Delta of its rows (BQ
  // floats each).
  static constexpr int SLOTB = 2 * TILEB + 2 * BQ * 4;
  static constexpr int LDS_BYTES = 2 * SLOTB;
  static_assert(BQ % 64 == 0 && NW >= 2, "the row statistics of a tile are 64-lane dword copies");
  // Fragment and staging addresses (FragOffT, Stager): at d = 256 the
  // XOR at each read and the periodic staging offsets (with one register
  // per read offset this kernel spills 80 to 104 bytes inside the loop).
  static constexpr bool XOR_ADDR = D >= 256;
  static constexpr bool PERIODIC_STAGE = D >= 256;
  using FragOff = typename Base::template FragOffT<XOR_ADDR>;
  using St = typename Base::template Stager<BQ, THREADS, PERIODIC_STAGE>;
  static_assert(!FragOff::XOR || SLOTB % ROWB == 0, "slot bases keep the fragment offsets' XOR bits");
  // dV and dK accumulators in AGPRs from d = 96 (one wave per SIMD: the
  // arch VGPRs hold the rest; see BwdBase::acc_mfma).
  static constexpr bool ACC_AGPR = D >= 96;
  // Software pipeline over the QBLK 32-row blocks of a tile: step j issues
  // the MFMAs of dV(j-1) and dK(j-1) (NG, u = 0 first), then of S(j+1) and
  // dP(j+1) (NSD, alternating), one at a time, each followed by its share of
  // the VALU work of block j (8 pairs: exponential, mask, dS, packing of P
  // and dS).
  static constexpr int NG = 4 * DB;
  static constexpr int NSD = 2 * DK;
  static constexpr int NPOS = NG + NSD;
  static constexpr int PF = D >= 256 ? 2 : 3;  // positions between a fragment's LDS read and its MFMA

  static __device__ __forceinline__ void run(const BwdParams& p, lds_char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    // Causal: the first key tiles (the most queries) first.
    const BwdItem item = bwd_work_item(p, blockIdx.x);
    const int ktile = item.step;
    const int bh = item.bh;
    const int n = p.n;
    const int k0 = ktile * BK;
    const int kw0 = k0 + 32 * wave;
    const int mykey = kw0 + (lane & 31);
    int klen = n, wl = kNoBound, wr = kNoBound;
    if constexpr (CAUSAL) wr = 0;
    if constexpr (GENERAL) {
      if (p.key_lens) klen = min(max(p.key_lens[bh / p.heads], 0), n);
      wl = p.wl;
      wr = p.wr;
    }

    const size_t slice = (size_t)bh * (size_t)n * D;
    const uint32_t bytes = (uint32_t)n * D * 2;
    // K and V rows at or past the key length (padding) are never read; their
    // dK and dV are 0 (every such key is hidden from every row).
    const auto rk = make_rsrc((const char*)p.k + slice * 2, (uint32_t)klen * D * 2);
    const auto rv = make_rsrc((const char*)p.v + slice * 2, (uint32_t)klen * D * 2);
    const auto rdk = make_rsrc((char*)p.dk + slice * 2, bytes);
    const auto rdv = make_rsrc((char*)p.dv + slice * 2, bytes);

    // K^T and V^T operands (lane: key mykey, dims 16ks + 8h .. +7).
    u32x4 kf[DK], vf[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      const int off = (mykey * D + 16 * ks + 8 * h) * 2;
      kf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      vf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }

    const FragOff fo(lane);
    const St st(tid);
    const u32x4 wq = rsrc_words(p.q, slice * 2, bytes);
    const u32x4 wdo = rsrc_words(p.dout, slice * 2, bytes);
    // The row statistics the dQ kernel left in the workspace.
    const u32x4 wd = rsrc_words(p.delta, (size_t)bh * n * 4, (uint32_t)n * 4);
    const u32x4 wl2 = rsrc_words(p.delta, ((size_t)p.bh + bh) * n * 4, (uint32_t)n * 4);

    f32x16 dv[DB], dk[DB];
    Base::template acc_zero<ACC_AGPR>(dv);
    Base::template acc_zero<ACC_AGPR>(dk);

    // Query tiles with a row that sees some key of the workgroup: [tfirst,
    // tend).  A tile takes the per-element mask when some (row, key) pair of
    // it is hidden: a key past the key length, a key after a row's right
    // bound (causal: after the row) or before its left bound.  Rows past N
    // load as zeros: Q, dO and both statistics 0, so P = 1 meets dO = 0 and
    // dP - Delta = 0, and the row adds exactly nothing.
    int rbeg = 0, rend = n;
    if constexpr (MASK != kMaskNone) {
      rbeg = max(0, k0 - wr);
      rend = min(n, k0 + BK + wl);  // k0 + BK - 1 + wl + 1
      if (k0 >= klen) rend = rbeg;  // every key of the workgroup is padding
    }
    const int tfirst = rbeg / BQ;
    const int tend = rend > rbeg ? (rend + BQ - 1) / BQ : tfirst;
    // The masked tiles are a prefix [tfirst, m1) (rows before the last key's
    // right bound: causal, rows before the last key) and a suffix [m2, tend)
    // (rows past the first key's left bound); all of them when the
    // workgroup holds a key past the key length.
    int m1 = tfirst, m2 = tend;
    if constexpr (MASK != kMaskNone) {
      const int rb = k0 + BK - 1 - wr;  // tiles starting before this row are masked
      m1 = min(tend, max(tfirst, rb > 0 ? (rb + BQ - 1) / BQ : tfirst));
      m2 = min(tend, max(m1, (int)(((int64_t)k0 + wl + 1) / BQ)));
      if (k0 + BK > klen) m1 = m2 = tend;
    }
    auto stage = [&](int t, const lds_char* dst) __attribute__((always_inline)) {
      st.stage(wq, dst, t * BQ);
      st.stage(wdo, dst + TILEB, t * BQ);
      // Wave 0: -LSE * log2(e) of the tile's rows; wave 1: -Delta.
#pragma unroll
      for (int half = 0; half < BQ / 64; ++half) {
        if (wave == 0) Base::dma4(wl2, dst + 2 * TILEB + half * 256, (t * BQ + 64 * half + lane) * 4);
        if (wave == 1) Base::dma4(wd, dst + 2 * TILEB + BQ * 4 + half * 256, (t * BQ + 64 * half + lane) * 4);
      }
    };
    auto tile = [&](int t, auto masked_c) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_c)::value;
      Base::dma_wait();
      __syncthreads();
      const int slot = Base::addr_of(lds) + ((t - tfirst) & 1) * SLOTB;
      const lds_char* sst = Base::at(slot) + 2 * TILEB;
      if (t + 1 < tend) stage(t + 1, lds + ((t + 1 - tfirst) & 1) * SLOTB);
      const int q0 = t * BQ;
      f32x16 sc[2], dp[2];      // S and dP - Delta of blocks of either parity
      f32x16 nl2[2];            // -LSE * log2(e) of the rows, accumulator order
      u32x4 pb[2][2], sb[2][2]; // packed P and dS of blocks of either parity
      // Row statistics of block qb in accumulator order: register r holds
      // tile row 32qb + 8(r/4) + 4h + r%4, four 16-byte reads.
      auto stats = [&](int qb, int which) __attribute__((always_inline)) -> f32x16 {
        f32x16 out;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = Base::lds_f4(sst + which * BQ * 4 + (32 * qb + 8 * g + 4 * h) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) out[4 * g + e] = x[e];
        }
        return out;
      };
      f32x16 ndel;  // -Delta of the block whose dP is being accumulated
      // A operand of MFMA `pos` of the step that works on block j.
      auto frag = [&](int j, int pos) __attribute__((always_inline)) -> u32x4 {
        if (pos < NG) {
          const int qb = j - 1, u = pos / (2 * DB), db = (pos % (2 * DB)) / 2;
          const int rows = (pos % 2 ? 0 : TILEB) + (qb * 32 + 16 * u) * ROWB;
          return Base::tr_frag(Base::at(fo.tr(slot, db, 0)) + rows, Base::at(fo.tr(slot, db, 1)) + rows);
        }
        const int qb = j + 1, ks = (pos - NG) / 2;
        return Base::lds16(Base::at(fo.plain(slot, ks)) + ((pos - NG) % 2 ? TILEB : 0) + qb * 32 * ROWB);
      };
      auto active = [&](int j, int pos) __attribute__((always_inline)) { return pos < NG ? j >= 1 : j + 1 < QBLK; };
      auto issue = [&](int j, int pos, const u32x4& a) __attribute__((always_inline)) {
        if (pos < NG) {
          const int qb = j - 1, u = pos / (2 * DB), db = (pos % (2 * DB)) / 2;
          if (pos % 2 == 0)
            Base::template acc_mfma<ACC_AGPR>(dv[db], a, pb[qb % 2][u]);
          else
            Base::template acc_mfma<ACC_AGPR>(dk[db], a, sb[qb % 2][u]);
        } else {
          const int qb = j + 1, ks = (pos - NG) / 2;
          if ((pos - NG) % 2 == 0)
            sc[qb % 2] = mfma32<BF16>(a, kf[ks], ks == 0 ? f32x16{} : sc[qb % 2]);
          else
            dp[qb % 2] = mfma32<BF16>(a, vf[ks], ks == 0 ? ndel : dp[qb % 2]);
        }
      };
      // VALU work of pair c of block j: registers 2c, 2c+1 (rows
      // q0 + 32j + 8(r/4) + 4h + r%4 against key mykey).
      auto pair = [&](int j, int c) __attribute__((always_inline)) {
        float x[2], y[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * c + e;
          x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j % 2][r], p.c2, nl2[j % 2][r]));
          if constexpr (MASKED) {
            const int row = q0 + 32 * j + 8 * (r >> 2) + 4 * h + (r & 3);
            if (mykey >= klen || mykey > row + wr || mykey < row - wl) x[e] = 0.f;
          }
          y[e] = x[e] * dp[j % 2][r];
        }
        pb[j % 2][c / 4][c % 4] = pack2<BF16>(x[0], x[1]);
        sb[j % 2][c / 4][c % 4] = pack2<BF16>(y[0], y[1]);
      };
      // Prologue: the statistics of block 0, S(0) and dP(0).
      nl2[0] = stats(0, 0);
      ndel = stats(0, 1);
      static_for<NG, NPOS>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pos = decltype(pc)::value;
        const u32x4 a = frag(-1, pos);
        issue(-1, pos, a);
      });
      static_for<0, QBLK>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j + 1 < QBLK) {
          nl2[(j + 1) % 2] = stats(j + 1, 0);
          ndel = stats(j + 1, 1);
        }
        u32x4 fr[NPOS];
        static_for<0, (PF < NPOS ? PF : NPOS)>([&](auto pc) __attribute__((always_inline)) {
          constexpr int pos = decltype(pc)::value;
          if (active(j, pos)) fr[pos] = frag(j, pos);
        });
        static_for<0, NPOS>([&](auto pc) __attribute__((always_inline)) {
          constexpr int pos = decltype(pc)::value;
          if constexpr (pos + PF < NPOS) {
            if (active(j, pos + PF)) fr[pos + PF] = frag(j, pos + PF);
          }
          if (active(j, pos)) issue(j, pos, fr[pos]);
          static_for<pos * 8 / NPOS, (pos + 1) * 8 / NPOS>(
              [&](auto cc) __attribute__((always_inline)) { pair(j, decltype(cc)::value); });
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      // Epilogue: dV(QBLK-1) and dK(QBLK-1).
      static_for<0, NG>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pos = decltype(pc)::value;
        const u32x4 a = frag(QBLK, pos);
        issue(QBLK, pos, a);
      });
    };
    if (tend > tfirst) stage(tfirst, lds);
    int t = tfirst;
    if constexpr (MASK != kMaskNone) {
      for (; t < m1; ++t) tile(t, std::true_type{});
    }
    for (; t < m2; ++t) tile(t, std::false_type{});
    if constexpr (GENERAL) {
      for (; t < tend; ++t) tile(t, std::true_type{});
    }
    Base::template settle<ACC_AGPR>(dv);
    Base::template settle<ACC_AGPR>(dk);
    Base::store_grad(rdv, dv, mykey, lane, 1.0f);
    Base::store_grad(rdk, dk, mykey, lane, p.scale);
  }
};

// Two waves per SIMD (256 registers each) up to d = 128, so that one wave's
// VALU work issues beside the other's MFMAs; one at d = 256.
template <int D, int NW, bool BF16, int MASK>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
    fa2_bwd_q_kernel(const BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds_generic[];
  Fa2BwdQ<D, NW, BF16, MASK>::run(
      p, (__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)lds_generic);
}

template <int D, int NW, bool BF16, int MASK>
__global__ void __launch_bounds__(NW * 64) fa2_bwd_kv_kernel(const BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds_generic[];
  Fa2BwdKV<D, NW, BF16, MASK>::run(
      p, (__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)lds_generic);
}

}  // namespace fa2
