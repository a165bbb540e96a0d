// FlashAttention-2 forward kernel for gfx950 (CDNA4), written for wave64 MFMA.
//
// What it computes (per batch b, head h, query row i):
//   O[i]   = sum_j P[i,j] V[j] / l_i,  P[i,j] = exp(scale * q_i.k_j - m_i),
//   l_i    = sum_j P[i,j],             LSE[i] = m_i + ln l_i
// over the keys visible to i (all keys, or j <= i when causal).  Method:
// "FlashAttention-2 MMA 代码学习" (chuoer47.github.io) step 1 (online (m, l)
// merge over key tiles), step 2 (split-Q: each wave owns whole query rows),
// step 3 (P stays in registers and feeds the second matrix product); and
// "第 15 章 FA2 前向：Tiling 与 Online Softmax" (yangyitao.com) §15.1 (outer loop
// over query tiles, grid over query tile x head x batch, deferred 1/l, LSE
// statistic), §15.3 (skeleton: causal tile bound, ragged-N zero fill and
// -inf column mask, -inf guards, out-of-range rows not stored), §15.5.1
// (double-buffered K/V staging with one barrier per tile).
//
// gfx950 mapping (a re-design, not a translation of the pages' mma.sync code):
//   * The score tile is computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16}: A = 32 keys x 16 dims (from LDS),
//     B = 16 dims x 32 queries (Q^T, resident in VGPRs for the whole kernel).
//     In the 32x32 accumulator, lane L holds query column L%32 and the 16 keys
//     8*(r/4) + 4*(L/32) + r%4 (r = accumulator register), so a query's row max
//     and row sum are in-lane reductions plus one exchange between the two
//     32-lane halves (v_permlane32_swap).
//   * The probabilities never leave the lane: registers r = 8u..8u+7 of a
//     32-key accumulator are exactly the B operand (16 keys x 32 queries) of
//     O^T += V^T P^T for k-step u, with keys ordered {16u+4h+e, 16u+8+4h+e}.
//   * V^T operands come from LDS with ds_read_b64_tr_b16, which transposes a
//     4-row x 16-column block of 16-bit values across 16 lanes; the rows each
//     lane group reads are chosen to match that key order.
//   * Software pipeline inside each wave: the MFMAs of S^T for tile j+1 are
//     issued before the softmax of tile j, so the matrix cores run while the
//     VALU computes exponentials; P V for tile j follows.
//   * The exponent base m is the running max, but it is only moved (and O and
//     l rescaled) when a tile's max exceeds it by more than 2^8 in the base-2
//     domain.  Any base gives the same softmax; this one keeps P <= 256 (exact
//     in fp16/bf16 up to the usual relative rounding) and drops the rescale
//     from almost every tile.  The pages rescale on every tile; the result is
//     the same.
//   * K and V tiles are staged global -> VGPR -> LDS, double-buffered, with
//     16-byte-chunk XOR swizzles so the MFMA operand reads do not collide in
//     LDS banks.  Out-of-range rows come back as zeros from buffer loads with a
//     range-checked resource (the pages' zero fill), and out-of-range stores
//     are dropped by the same check.
//   * The grid is one workgroup per (query tile, batch*head); consecutive
//     workgroup ids walk the heads first, so with B*H a multiple of 8 every
//     head stays on one XCD (workgroups are dealt to the 8 XCDs round robin)
//     and its K/V stay in that XCD's L2.  Causal grids issue the longest query
//     tiles first.
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
};

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle, offsets range-checked against num_records).
constexpr int kRsrcWord3 = 0x00020000;

// The exponent base moves only when a row's tile max exceeds it by more than
// this (base-2 units), so probabilities stay below 2^kRebase.
constexpr float kRebase = 8.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
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

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ f16x2 ones_f16x2() { return f16x2{(_Float16)1.0f, (_Float16)1.0f}; }

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

// LDS layouts.  A K or V tile is BC rows (keys) of D 16-bit values, stored as
// 16-byte chunks; chunk c of row r sits at chunk position c ^ swz(r).  The XOR
// only permutes chunks inside aligned groups of 8, so a row stays in place.
//  * K rows are read 16 bytes per lane by 32 consecutive rows at one chunk:
//    rows r..r+7 must land on 8 different chunk positions.
//  * V rows are read 8 bytes per lane by ds_read_b64_tr_b16: a 16-lane group
//    covers 4 consecutive rows x 2 adjacent chunks; 2*(r%4) spreads them over
//    all 8 positions.
__device__ __forceinline__ int swz_k(int row) { return row & 7; }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

template <int D, int BC, int NW, int QB, bool BF16, bool CAUSAL>
struct Fa2Fwd {
  static constexpr int THREADS = NW * 64;
  static constexpr int QW = 32 * QB;             // query rows per wave
  static constexpr int BR = NW * QW;             // query rows per workgroup
  static constexpr int KB = BC / 32;             // 32-key blocks per tile
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  static constexpr int DK = D / 16;              // 16-deep k-steps of S^T = K Q^T
  static constexpr int ROWB = D * 2;             // bytes per K/V row
  static constexpr int TILEB = BC * ROWB;        // bytes per K (or V) tile
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / THREADS; // chunks per thread per tile (each of K, V)
  static constexpr int LDS_BYTES = 4 * TILEB;    // K[0], K[1], V[0], V[1]
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BC * CPR) % THREADS == 0 && CPT >= 1, "staging split");
  // Every LDS access below is a lane base register plus a compile-time
  // offset; keeping the whole LDS image under 64 KiB lets the offsets ride in
  // the instruction's 16-bit immediate.
  static_assert(LDS_BYTES <= 65536, "LDS image must fit the ds immediate offset");

  typedef __attribute__((address_space(3))) char lds_char;

  // Lane-constant LDS byte offsets (relative to the K or V buffer base).
  struct LdsOffsets {
    int k[DK];     // K^T operand of k-step ks for key block 0 (block kb adds kb*32 rows)
    int v[DB];     // V^T operand rows 32*db..: keys 4h+e of a 16-key group (+8 rows: second read)
    int kst[CPT];  // staging store of chunk j, K layout
    int vst[CPT];  // staging store of chunk j, V layout
    int gld[CPT];  // global byte offset of chunk j inside a tile
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
        for (int i = 0; i < KG; ++i) a[i] = *(const __attribute__((address_space(3))) u32x4*)(sk + off.k[g + i] + kb * 32 * ROWB);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int i = 0; i < KG; ++i)
            out.s[qb][kb] = mfma32<BF16>(a[i], qf[qb][g + i], (g + i == 0) ? f32x16{} : out.s[qb][kb]);
        }
      }
    }
  }

  // Online softmax of one tile: updates the exponent base m, the lane's share
  // of l and (rarely) rescales O; turns the scores into packed probabilities
  // laid out as the B operands of O^T += V^T P^T.
  template <bool MASK>
  static __device__ __forceinline__ void softmax(Scores& sc, u32x4 (&pb)[QB][KB][2], float (&m)[QB],
                                                 float (&l)[QB], f32x16 (&o)[QB][DB], float c2,
                                                 int lane, int k0, int qw0, int n) {
    const int half = lane >> 5;
    const float ninf = -__builtin_inff();
    if constexpr (MASK) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw0 + 32 * qb + (lane & 31);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool hide = (key >= n) || (CAUSAL && key > qrow);
            sc.s[qb][kb][r] = hide ? ninf : sc.s[qb][kb][r];
          }
        }
      }
    }
    bool rebase = false;
    float mt[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Two independent max chains, merged at the end.
      float ma = ninf, mb = ninf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          ma = __builtin_fmaxf(__builtin_fmaxf(ma, sc.s[qb][kb][r]), sc.s[qb][kb][r + 1]);
          mb = __builtin_fmaxf(__builtin_fmaxf(mb, sc.s[qb][kb][r + 2]), sc.s[qb][kb][r + 3]);
        }
      }
      float mx = __builtin_fmaxf(ma, mb);
      float lo, hi;
      halves(mx, lo, hi);
      mx = __builtin_fmaxf(lo, hi);
      mt[qb] = (mx == ninf) ? ninf : mx * c2;
      rebase |= mt[qb] > m[qb] + kRebase;
    }
    // Wave-uniform decision: move the base of every row whose max grew.
    if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = __builtin_fmaxf(m[qb], mt[qb]);
        // A row that has seen only masked keys keeps -inf (its sums are zero).
        const float alpha = (m_new == ninf) ? 1.f : __builtin_amdgcn_exp2f(m[qb] - m_new);
        m[qb] = m_new;
        l[qb] *= alpha;
        // In-place multiply: keeps O in the same registers on both sides of
        // this rarely taken branch.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = o[qb][db][r];
            asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(alpha));
            o[qb][db][r] = x;
          }
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mb = m[qb];
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc.s[qb][kb][r], c2, -mb));
          if constexpr (MASK) p = (sc.s[qb][kb][r] == ninf) ? 0.f : p;
          sc.s[qb][kb][r] = p;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = sc.s[qb][kb][8 * u + 2 * e], p1 = sc.s[qb][kb][8 * u + 2 * e + 1];
            pb[qb][kb][u][e] = pack2<BF16>(p0, p1);
            if constexpr (BF16) {
              // fp32 sum of the unrounded probabilities.
              sa += p0;
              sb += p1;
            } else {
              // fp16: sum of the rounded probabilities with one dot product
              // against (1, 1); P V uses the same rounded values.  The packed
              // word goes through a scalar first: bit-casting a vector element
              // in place miscompiles (always reads element 0) in this clang.
              const uint32_t w = pb[qb][kb][u][e];
              if (e & 1)
                sb = __builtin_amdgcn_fdot2(as_f16x2(w), ones_f16x2(), sb, false);
              else
                sa = __builtin_amdgcn_fdot2(as_f16x2(w), ones_f16x2(), sa, false);
            }
          }
        }
      }
      l[qb] += sa + sb;
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
        const int rows = (kb * 32 + 16 * u) * ROWB;
#pragma unroll
        for (int g = 0; g < DB; g += VG) {
          u32x4 a[VG];
#pragma unroll
          for (int i = 0; i < VG; ++i) {
            const s16x4 va = lds_read_tr16(sv + off.v[g + i] + rows);
            const s16x4 vb = lds_read_tr16(sv + off.v[g + i] + rows + 8 * ROWB);
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

    // Work item: heads vary fastest; causal grids take the longest tiles first.
    const int wg = blockIdx.x;
    const int bh = wg % p.bh;
    const int t = wg / p.bh;
    const int qtile = CAUSAL ? (p.n_qtiles - 1 - t) : t;
    const int n = p.n;
    const int q0 = qtile * BR;
    const int qw0 = q0 + wave * QW;  // first query of this wave

    const size_t slice = (size_t)bh * (size_t)n * D;  // elements before this head
    const uint32_t slice_bytes = (uint32_t)n * D * 2;
    const auto rq = make_rsrc((const char*)p.q + slice * 2, slice_bytes);
    const auto rk = make_rsrc((const char*)p.k + slice * 2, slice_bytes);
    const auto rv = make_rsrc((const char*)p.v + slice * 2, slice_bytes);
    const auto ro = make_rsrc((char*)p.o + slice * 2, slice_bytes);
    const auto rl = make_rsrc(p.lse + (size_t)bh * n, (uint32_t)n * 4);

    // Q^T operands: for k-step s, lane holds Q[row][16s + 8*half .. +7].
    u32x4 qf[QB][DK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + 32 * qb + (lane & 31);
#pragma unroll
      for (int s = 0; s < DK; ++s) {
        qf[qb][s] = __builtin_amdgcn_raw_buffer_load_b128(rq, (qrow * D + 16 * s + 8 * half) * 2, 0, 0);
        qf[qb][s] ^= p.q_sign;
      }
    }

    // Lane-constant LDS offsets.
    LdsOffsets off;
    {
      const int row = lane & 31;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) off.k[ks] = row * ROWB + (((2 * ks + half) ^ swz_k(row)) << 4);
      // V^T transposed reads: lane group g = lane/16 serves A rows (dims)
      // 16*(g%2) + lane%16 for key half g/2; as a source, lane 16g + 4e + u
      // reads key row 4*(g/2) + e at dims 16*(g%2) + 4u .. +3.  Rows 32kb+16u
      // (+8) are added as immediates; they keep key%4 and so the swizzle.
      const int g = lane >> 4;
      const int key = 4 * (g >> 1) + ((lane >> 2) & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dim = 32 * db + 16 * (g & 1) + 4 * (lane & 3);
        off.v[db] = key * ROWB + (((dim >> 3) ^ swz_v(key)) << 4) + ((dim & 7) << 1);
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + THREADS * j;
        const int r = c / CPR, col = c % CPR;
        off.kst[j] = r * ROWB + ((col ^ swz_k(r)) << 4);
        off.vst[j] = r * ROWB + ((col ^ swz_v(r)) << 4);
        off.gld[j] = (r * D + col * 8) * 2;
      }
    }

    const float c2 = p.scale_log2;
    f32x16 o[QB][DB];
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m[qb] = -__builtin_inff();  // exponent base (base-2 domain)
      l[qb] = 0.f;                // this lane's share of the row sum
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
    }

    const int kend = CAUSAL ? min(n, q0 + BR) : n;
    const int ntiles = (kend + BC - 1) / BC;

    // Staging of tile j: global -> registers (soffset = tile start), then LDS.
    u32x4 stk[CPT], stv[CPT];
    auto load = [&](int j) {
      const int base = j * TILEB;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        stk[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off.gld[i], base, 0);
        stv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off.gld[i], base, 0);
      }
    };
    auto store = [&](auto buf) {
      constexpr int B = decltype(buf)::value;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        *(__attribute__((address_space(3))) u32x4*)(lds + B * TILEB + off.kst[i]) = stk[i];
        *(__attribute__((address_space(3))) u32x4*)(lds + (2 + B) * TILEB + off.vst[i]) = stv[i];
      }
    };

    // A wave takes part in tile j if some key of it is visible to some of its rows.
    auto active = [&](int j) { return !CAUSAL || j * BC <= qw0 + QW - 1; };
    // Tile j needs per-element masking (ragged tail or causal diagonal).
    auto masked = [&](int j) { return (j * BC + BC > n) || (CAUSAL && j * BC + BC - 1 > qw0); };

    // Tile j lives in buffer j%2 (K and V).  Its successor is loaded from
    // global memory at the top of iteration j and written to the other buffer
    // at the bottom; that buffer was last read in iteration j-1, before the
    // barrier that ended it.
    auto step = [&](int j, auto buf) {
      constexpr int B = decltype(buf)::value;
      const bool more = j + 1 < ntiles;
      if (more) load(j + 1);
      if (active(j)) {
        Scores sc;
        scores(lds + B * TILEB, off, qf, sc);
        u32x4 pb[QB][KB][2];
        if (masked(j))
          softmax<true>(sc, pb, m, l, o, c2, lane, j * BC, qw0, n);
        else
          softmax<false>(sc, pb, m, l, o, c2, lane, j * BC, qw0, n);
        pv(lds + (2 + B) * TILEB, off, pb, o);
      }
      if (more) store(std::integral_constant<int, 1 - B>{});
      __syncthreads();
    };

    load(0);
    store(std::integral_constant<int, 0>{});
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
      step(j, std::integral_constant<int, 0>{});
      if (j + 1 < ntiles) step(j + 1, std::integral_constant<int, 1>{});
    }

    // Epilogue: combine the two halves' partial sums, divide once, store.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + 32 * qb + (lane & 31);
      float l_lo, l_hi;
      halves(l[qb], l_lo, l_hi);
      const float l_tot = l_lo + l_hi;
      const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack2<BF16>(o[qb][db][4 * g + 0] * inv, o[qb][db][4 * g + 1] * inv);
          w[1] = pack2<BF16>(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
          const int dim = 32 * db + 8 * g + 4 * half;
          __builtin_amdgcn_raw_buffer_store_b64(w, ro, (qrow * D + dim) * 2, 0, 0);
        }
      }
      if (half == 0) {
        const float lse = (l_tot > 0.f) ? (m[qb] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                        : __builtin_inff();
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qrow * 4, 0, 0);
      }
    }
  }
};

template <int D, int BC, int NW, int QB, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 1) fa2_fwd_kernel(const Params p) {
  extern __shared__ __attribute__((aligned(16))) char lds_generic[];
  Fa2Fwd<D, BC, NW, QB, BF16, CAUSAL>::run(
      p, (__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)lds_generic);
}

}  // namespace fa2
