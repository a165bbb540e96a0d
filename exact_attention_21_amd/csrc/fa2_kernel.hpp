// FlashAttention-2 forward kernel for gfx950 (CDNA4), written for wave64 MFMA.
//
// What it computes (per batch b, head h, query row i):
//   O[i]   = sum_j P[i,j] V[j] / l_i,  P[i,j] = exp(scale * q_i.k_j - m_i)
//   LSE[i] = m_i + ln l_i
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Exchange a float with the lane 32 positions away and combine: returns the
// pair (value of the lower-half lane, value of the upper-half lane), identical
// in both lanes of the pair.
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

// Two fp32 values -> one dword of two 16-bit values, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

template <int D, int BC, int NW, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 1) fa2_fwd_kernel(const Params p) {
  constexpr int THREADS = NW * 64;
  constexpr int BR = NW * 32;             // query rows per workgroup (32 per wave)
  constexpr int KB = BC / 32;             // 32-key blocks per tile
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int DK = D / 16;              // 16-deep k-steps of S^T = K Q^T
  constexpr int ROWB = D * 2;             // bytes per K/V row
  constexpr int TILEB = BC * ROWB;        // bytes per K (or V) tile
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int CPT = BC * CPR / THREADS; // chunks per thread per tile (each of K, V)
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BC * CPR) % THREADS == 0 && CPT >= 1, "staging split");

  extern __shared__ __attribute__((aligned(16))) char lds[];  // [2 buffers][K | V][BC][D]

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
  const int qw0 = q0 + wave * 32;          // first query of this wave
  const int qrow = qw0 + (lane & 31);      // this lane's query

  const size_t slice = (size_t)bh * (size_t)n * D;  // elements before this head
  const uint32_t slice_bytes = (uint32_t)n * D * 2;
  const auto rq = make_rsrc((const char*)p.q + slice * 2, slice_bytes);
  const auto rk = make_rsrc((const char*)p.k + slice * 2, slice_bytes);
  const auto rv = make_rsrc((const char*)p.v + slice * 2, slice_bytes);
  const auto ro = make_rsrc((char*)p.o + slice * 2, slice_bytes);
  const auto rl = make_rsrc(p.lse + (size_t)bh * n, (uint32_t)n * 4);

  // Q^T operand: for k-step s, lane holds Q[qrow][16s + 8*half .. +7].
  u32x4 qf[DK];
#pragma unroll
  for (int s = 0; s < DK; ++s) {
    qf[s] = __builtin_amdgcn_raw_buffer_load_b128(rq, (qrow * D + 16 * s + 8 * half) * 2, 0, 0);
    qf[s] ^= p.q_sign;
  }

  const float c2 = p.scale_log2;
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff();  // running max of c2*s (base-2 domain)
  float l_run = 0.f;                // this lane's share of the running sum

  const int kend = CAUSAL ? min(n, q0 + BR) : n;
  const int ntiles = (kend + BC - 1) / BC;

  // Staging: thread handles chunks c = tid + THREADS*j of each tile.
  u32x4 stk[CPT], stv[CPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + THREADS * j;
      const int row = c / CPR, col = c % CPR;
      const int off = ((k0 + row) * D + col * 8) * 2;
      stk[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      stv[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
    char* sk = lds + buf * 2 * TILEB;
    char* sv = sk + TILEB;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + THREADS * j;
      const int row = c / CPR, col = c % CPR;
      *(u32x4*)(sk + row * ROWB + ((col ^ swz_k(row)) << 4)) = stk[j];
      *(u32x4*)(sv + row * ROWB + ((col ^ swz_v(row)) << 4)) = stv[j];
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  // Per-lane constants for the V^T transposed reads: lane group g = lane/16
  // serves A rows (dims) 16*(g%2) + lane%16 for key half g/2; as a source,
  // lane 16g + 4e + u reads key row (4*(g/2) + e) at dims 16*(g%2) + 4u .. +3.
  const int tr_g = lane >> 4;
  const int tr_key = 4 * (tr_g >> 1) + ((lane >> 2) & 3);
  const int tr_dim = 16 * (tr_g & 1) + 4 * (lane & 3);

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * BC;
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile(k0 + BC);

    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    if (active) {
      const char* sk = lds + buf * 2 * TILEB;
      const char* sv = sk + TILEB;

      // S^T for each 32-key block.
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        const int row = kb * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          const int col = 2 * ks + half;
          const u32x4 a = *(const u32x4*)(sk + row * ROWB + ((col ^ swz_k(row)) << 4));
          s[kb] = mfma32<BF16>(a, qf[ks], s[kb]);
        }
      }

      // Mask (ragged tail and causal diagonal only).
      const bool need_mask = (k0 + BC > n) || (CAUSAL && k0 + BC - 1 > qw0);
      const float ninf = -__builtin_inff();
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool hide = (key >= n) || (CAUSAL && key > qrow);
            s[kb][r] = hide ? ninf : s[kb][r];
          }
        }
      }

      // Row max of the raw scores (scale is >= 0 after the Q sign fold).
      float mx = ninf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
      }
      {
        float lo, hi;
        halves(mx, lo, hi);
        mx = __builtin_fmaxf(lo, hi);
      }
      const float mxs = (mx == ninf) ? ninf : mx * c2;
      const float m_new = __builtin_fmaxf(m_run, mxs);
      // A row that has seen only masked keys keeps -inf; use 0 as the base
      // so that exp2(-inf - (-inf)) is never formed.
      const float m_use = (m_new == ninf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -m_use));
          if (need_mask) pv = (s[kb][r] == ninf) ? 0.f : pv;
          s[kb][r] = pv;
          lsum += pv;
        }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;

      // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 pb;
#pragma unroll
          for (int e = 0; e < 4; ++e) pb[e] = pack2<BF16>(s[kb][8 * u + 2 * e], s[kb][8 * u + 2 * e + 1]);
          const int key_a = kb * 32 + 16 * u + tr_key;
          const int key_b = key_a + 8;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int dim = 32 * db + tr_dim;
            const int ca = dim >> 3;
            const char* pa = sv + key_a * ROWB + ((ca ^ swz_v(key_a)) << 4) + ((dim & 7) << 1);
            const char* pbp = sv + key_b * ROWB + ((ca ^ swz_v(key_b)) << 4) + ((dim & 7) << 1);
            const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) const char*)pa);
            const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) const char*)pbp);
            u32x4 a;
            a[0] = __builtin_bit_cast(u32x2, va)[0];
            a[1] = __builtin_bit_cast(u32x2, va)[1];
            a[2] = __builtin_bit_cast(u32x2, vb)[0];
            a[3] = __builtin_bit_cast(u32x2, vb)[1];
            o[db] = mfma32<BF16>(a, pb, o[db]);
          }
        }
      }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: combine the two halves' partial sums, divide once, store.
  float l_lo, l_hi;
  halves(l_run, l_lo, l_hi);
  const float l_tot = l_lo + l_hi;
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack2<BF16>(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      w[1] = pack2<BF16>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      const int dim = 32 * db + 8 * g + 4 * half;
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, (qrow * D + dim) * 2, 0, 0);
    }
  }
  if (half == 0) {
    const float lse = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                    : __builtin_inff();
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qrow * 4, 0, 0);
  }
}

}  // namespace fa2
