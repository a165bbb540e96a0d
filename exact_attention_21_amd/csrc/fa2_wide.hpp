// FlashAttention-2 forward for head dims 512 and 1024 on gfx950.
//
// The pages reach large head dims by tiling the head dimension as well as the
// keys ("flash_attn_mma_stages_split_q_tiling_qk", the third page: Q and K
// staged as d-slices, V as [16, d] slices, so that shared memory stays
// O(16 d)).  On gfx950 a whole 32-key tile of K is 32 KiB at d = 512 and
// 64 KiB at d = 1024, so the four-slot K and V rings of the main kernel do
// not fit the 160 KiB LDS.  This kernel keeps the main kernel's register
// design (S^T = K Q^T on 32x32x16 MFMAs, P kept in registers as the B
// operand of O^T += V^T P^T, Q^T in VGPRs for the whole kernel, O^T in
// AGPRs) and streams K and V through LDS in 128-dim chunks instead:
//
//   * A key tile is 2C chunks of 32 keys x 128 dims (8 KiB): K chunks
//     0..C-1, then V chunks 0..C-1 (C = d / 128).  A chunk has exactly the
//     layout of a d = 128 tile of the main kernel (256-byte rows, the same
//     conflict-free K and V swizzles), loaded straight from global memory
//     into an 8-slot ring, 7 chunks ahead, one barrier per chunk.
//   * S of a tile accumulates over its K chunks; its softmax runs once the
//     last K chunk is in; P then meets the V chunks.
//   * One wave per SIMD (4 per workgroup), so that a wave has all 512
//     registers: d = 512: each wave owns 32 rows, computes all of S and owns
//     all 512 output dims (16 AGPR blocks, 256 AGPRs; Q^T is 128 VGPRs);
//     128 rows per workgroup.  d = 1024: two waves per 32 rows (64 rows per
//     workgroup).  Each wave of a pair takes half the k-steps of every K
//     chunk and half the output dims of every V chunk (the same register
//     budget); the two partial score tiles are added through LDS, in either
//     order, which gives both waves bit-identical scores and so the same
//     softmax.
//   * Exponent base: fixed at a row's first visible scores and moved only
//     when a later tile's row max exceeds it by more than 8 (log2 units), so
//     every probability is at most 2^8 and O is rarely rescaled; the moves
//     follow the online (m, l) update of the pages.
//
// Masks, ragged N, the scale's sign, LSE and the fully-masked-row rules are
// those of the main kernel (fa2_kernel.hpp).
#pragma once

#include "fa2_kernel.hpp"

namespace fa2 {

template <int D, bool BF16, int MASK>
struct Fa2Wide {
  static_assert(D == 512 || D == 1024, "chunked kernel: d = 512 or 1024");
  static constexpr bool CAUSAL = MASK == kMaskCausal;
  static constexpr bool GENERAL = MASK == kMaskGeneral;
  static constexpr int BC = 32;                             // keys per tile
  static constexpr int CW = 128;                            // dims per chunk
  static constexpr int C = D / CW;                          // chunks per K (or V) tile
  static constexpr bool PAIR = D == 1024;                   // two waves per 32 query rows
  static constexpr int NW = 4;
  static constexpr int THREADS = NW * 64;
  static constexpr int BR = (PAIR ? NW / 2 : NW) * 32;      // query rows per workgroup
  static constexpr int KS = PAIR ? 4 : 8;                   // k-steps of a chunk per wave
  static constexpr int VB = PAIR ? 2 : 4;                   // 32-dim output blocks of a chunk per wave
  static constexpr int QK = C * KS;                         // Q^T operands per wave
  static constexpr int OB = C * VB;                         // O^T blocks per wave
  static constexpr int ROWB = CW * 2;                       // bytes per chunk row
  static constexpr int SLOTB = BC * ROWB;                   // bytes per chunk
  static constexpr int RING = 8;                            // chunk slots
  static constexpr int PF = RING - 1;                       // chunks loaded ahead
  static constexpr int CPT = SLOTB / 16 / THREADS;          // 16-byte loads per thread per chunk
  static constexpr int STEPS = 2 * C;                       // chunks per key tile
  static constexpr int XCH_BYTES = PAIR ? NW * 64 * 64 : 0;  // partial scores: 16 floats per lane
  static constexpr int LDS_BYTES = RING * SLOTB + XCH_BYTES;
  static constexpr bool LSE_FP32 = BF16;  // as in the main kernel
  static_assert(CPT >= 1 && CPT * THREADS * 16 == SLOTB, "chunk staging");
  static_assert(STEPS % RING == 0, "a tile's chunks use fixed ring slots");
  static_assert(QK * 16 * (PAIR ? 2 : 1) == D && OB * 32 * (PAIR ? 2 : 1) == D, "work split");

  typedef __attribute__((address_space(3))) char lds_char;

  // Largest step of a row max above the current base that is absorbed
  // without moving it (probabilities stay <= 2^8).
  static constexpr float kMargin = 8.0f;

  struct Ctx {
    u32x4 wk, wv;       // K and V buffer descriptors (raw words, for the inline-asm loads)
    lds_char* lds;
    int koff[KS];       // K^T operand of the wave's k-step ks of a chunk
    int voff[VB];       // V^T operand rows of the wave's output block vb of a chunk
    int gdk[CPT];       // global byte offset (within a chunk column) of the K piece a lane loads
    int gdv[CPT];       // the same for V
    int dma;            // this wave's first LDS byte of a chunk (lane L adds 16 L)
    int tfirst;         // first key tile of the workgroup
    int qw0, n, wl, wr, lane;
    float c2;
    // A wave takes part in tile j if some key of it is visible to some of its rows.
    __device__ __forceinline__ bool active(int j) const {
      if constexpr (CAUSAL) return j * BC <= qw0 + 31;
      if constexpr (GENERAL) return j * BC < n && j * BC <= qw0 + 31 + wr && j * BC + BC - 1 >= qw0 - wl;
      return true;
    }
    // Tile j needs per-element masking.
    __device__ __forceinline__ bool masked(int j) const {
      if constexpr (GENERAL) return (j * BC + BC > n) || (j * BC + BC - 1 > qw0 + wr) || (j * BC < qw0 + 31 - wl);
      return (j * BC + BC > n) || (CAUSAL && j * BC + BC - 1 > qw0);
    }
  };

  struct State {
    u32x4 qf[QK];     // Q^T operands
    f32x16 o[OB];     // O^T accumulators (AGPRs)
    f32x16 s;         // S^T of the current tile
    u32x4 pb[2];      // P of the current tile: B operands of the two 16-key k-steps
    float m;          // exponent base of this lane's query row (base 2, scaled)
    float lr;         // this lane's share of the sum of the rounded probabilities
    float lu;         // bf16: the same for the unrounded ones
  };

  // Wait states after the inline-asm output MFMAs before the compiler reads
  // their accumulators: an MFMA result latency, then empty statements that
  // claim to modify every accumulator, so no read of O is scheduled above the
  // wait (see Fa2Fwd::settle_o).
  static __device__ __forceinline__ void settle_o(State& st) {
    asm volatile("s_nop 7\n s_nop 7\n s_nop 3");
#pragma unroll
    for (int ob = 0; ob < OB; ++ob) asm volatile("" : "+a"(st.o[ob]));
  }

  static __device__ __forceinline__ void dma16(const u32x4& rsrc, const lds_char* dst, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n s_nop 0\n buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voffset), "s"(rsrc) : "memory", "m0");
  }

  // Chunk g of the workgroup's stream (tile tfirst + g / STEPS, K chunk g % STEPS
  // or V chunk g % STEPS - C) into ring slot g % RING.  Rows past the keys
  // present read as zeros.
  template <int GS>
  static __device__ __forceinline__ void load_chunk(const Ctx& cx, int t) {
    constexpr int S = GS % STEPS;
    constexpr bool ISV = S >= C;
    constexpr int CI = ISV ? S - C : S;
    constexpr int SLOT = GS % RING;
    const int tile = cx.tfirst + t + GS / STEPS;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      dma16(ISV ? cx.wv : cx.wk, cx.lds + SLOT * SLOTB + cx.dma + THREADS * 16 * i,
            (ISV ? cx.gdv[i] : cx.gdk[i]) + CI * CW * 2 + tile * BC * D * 2);
  }
  template <int G>
  static __device__ __forceinline__ void prologue_loads(const Ctx& cx) {
    if constexpr (G < PF) {
      load_chunk<G>(cx, 0);
      prologue_loads<G + 1>(cx);
    }
  }

  static __device__ __forceinline__ s16x4 tr16(const lds_char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  }

  // Per-element mask of the current tile (see fa2_kernel.hpp mask_scores).
  static __device__ __forceinline__ void mask_scores(const Ctx& cx, f32x16& s, int k0) {
    const int half = cx.lane >> 5;
    const int qrow = cx.qw0 + (cx.lane & 31);
    const float ninf = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool hide = (key >= cx.n) || (CAUSAL && key > qrow) ||
                        (GENERAL && (key > qrow + cx.wr || key < qrow - cx.wl));
      s[r] = hide ? ninf : s[r];
    }
  }

  // Softmax of tile j: move the base if a row max outgrew it, then the
  // probabilities (hidden keys exactly 0), packed into P, and the row sums.
  static __device__ __forceinline__ void softmax(const Ctx& cx, State& st, int j) {
    if (__builtin_expect(!cx.active(j) || cx.masked(j), 0)) mask_scores(cx, st.s, j * BC);
    const float ninf = -__builtin_inff();
    float mx = ninf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, st.s[r]);
    float lo, hi;
    halves(mx, lo, hi);
    mx = __builtin_fmaxf(lo, hi);
    const float mt = (mx == ninf) ? ninf : mx * cx.c2;
    const bool grow = mt > st.m + kMargin;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
      // O was last written by output MFMAs the compiler does not track.
      settle_o(st);
      const float m_new = grow ? mt : st.m;
      const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 from the unseen base
#pragma unroll
      for (int ob = 0; ob < OB; ++ob) {
        asm volatile("" : "+a"(st.o[ob]));
        st.o[ob] *= alpha;
        asm volatile("" : "+a"(st.o[ob]));
      }
      st.lr *= alpha;
      if constexpr (LSE_FP32) st.lu *= alpha;
      st.m = m_new;
    }
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += 2) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[r0], cx.c2, -st.m));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[r0 + 1], cx.c2, -st.m));
      p0 = st.s[r0] == ninf ? 0.f : p0;  // also where scale 0 meets a hidden key
      p1 = st.s[r0 + 1] == ninf ? 0.f : p1;
      const uint32_t w = pack2<BF16>(p0, p1);
      st.pb[r0 >> 3][(r0 & 7) >> 1] = w;
      // The row sum of the values the output MFMA multiplies.
      float q0, q1;
      if constexpr (BF16) {
        q0 = __uint_as_float(w << 16);
        q1 = __uint_as_float(w & 0xffff0000u);
      } else {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        q0 = (float)h[0];
        q1 = (float)h[1];
      }
      st.lr += q0 + q1;
      if constexpr (LSE_FP32) st.lu += p0 + p1;
    }
    // The output MFMAs that read P are inline asm, for which the compiler
    // inserts no wait states after a VALU write of an operand: keep the
    // packing here, ahead of the next chunk's loads and LDS reads, instead of
    // letting it sink next to the first output MFMA.
    asm volatile("" : "+v"(st.pb[0]), "+v"(st.pb[1]));
  }

  // Step S of tile t (chunk g = t * STEPS + S of the stream, ring slot S % RING).
  template <int S>
  static __device__ __forceinline__ void step(const Ctx& cx, State& st, int t, lds_char* xch) {
    constexpr int SLOT = S % RING;
    load_chunk<S + PF>(cx, t);
    const lds_char* sl = cx.lds + SLOT * SLOTB;
    if constexpr (S < C) {
      // S^T += K chunk S . Q^T over this wave's k-steps of the chunk.
      u32x4 a[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ks] = *(const __attribute__((address_space(3))) u32x4*)(sl + cx.koff[ks]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st.s = mfma32<BF16>(a[ks], st.qf[S * KS + ks], (S == 0 && ks == 0) ? f32x16{} : st.s);
      if constexpr (PAIR && S == C - 1) {
        // This wave's partial scores, for the other wave of the pair, as
        // [register group][lane] so that each 16-lane quarter of a write
        // covers 256 contiguous bytes (all 64 banks once).
        auto* x = (__attribute__((address_space(3))) f32x4*)(xch + (threadIdx.x >> 6) * 4096);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[i * 64 + cx.lane] = f32x4{st.s[4 * i], st.s[4 * i + 1], st.s[4 * i + 2], st.s[4 * i + 3]};
      }
    } else {
      // O^T += V^T (chunk S - C) . P^T for this wave's output blocks of the chunk.
      constexpr int CI = S - C;
      u32x4 a[2][VB];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const s16x4 va = tr16(sl + cx.voff[vb] + 16 * u * ROWB);
          const s16x4 vc = tr16(sl + cx.voff[vb] + (16 * u + 8) * ROWB);
          a[u][vb] = u32x4{__builtin_bit_cast(u32x2, va)[0], __builtin_bit_cast(u32x2, va)[1],
                           __builtin_bit_cast(u32x2, vc)[0], __builtin_bit_cast(u32x2, vc)[1]};
        }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) mfma32_acc_agpr<BF16>(st.o[CI * VB + vb], a[u][vb], st.pb[u]);
    }
    // Chunk g + 1 has landed once at most the PF - 1 newer chunks are in flight.
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((PF - 1) * CPT) : "memory");
    __syncthreads();
    if constexpr (S == C - 1) {
      if constexpr (PAIR) {
        const auto* x = (const __attribute__((address_space(3))) f32x4*)(xch + ((threadIdx.x >> 6) ^ 1) * 4096);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 y = x[i * 64 + cx.lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) st.s[4 * i + e] += y[e];
        }
      }
      softmax(cx, st, cx.tfirst + t);
    }
  }
  template <int S>
  static __device__ __forceinline__ void steps(const Ctx& cx, State& st, int t, lds_char* xch) {
    if constexpr (S < STEPS) {
      step<S>(cx, st, t, xch);
      steps<S + 1>(cx, st, t, xch);
    }
  }

  static __device__ __forceinline__ void run(const Params& p, lds_char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int pw = PAIR ? (wave & 1) : 0;   // the wave's half of each chunk (pairs)
    const int rw = PAIR ? (wave >> 1) : wave;

    const WorkItem item = work_item(p, blockIdx.x);
    const int bh = item.bh;
    const int qtile = MASK != kMaskNone ? (p.n_qtiles - 1 - item.step) : item.step;
    const int n = p.n;
    const int q0 = qtile * BR;
    const int qw0 = q0 + rw * 32;
    const int qrow = qw0 + (lane & 31);

    const size_t slice = (size_t)bh * (size_t)n * D;
    const uint32_t slice_bytes = (uint32_t)n * D * 2;
    const auto rq = make_rsrc((const char*)p.q + slice * 2, slice_bytes);
    const auto ro = make_rsrc((char*)p.o + slice * 2, slice_bytes);
    const auto rl = make_rsrc(p.lse + (size_t)bh * n, (uint32_t)n * 4);

    State st;
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) {
      const int ksg = (kk / KS) * 8 + pw * KS + kk % KS;  // 16-dim k-step of the head dim
      st.qf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, (qrow * D + 16 * ksg + 8 * half) * 2, 0, 0);
      st.qf[kk] ^= p.q_sign;
    }
#pragma unroll
    for (int ob = 0; ob < OB; ++ob) st.o[ob] = f32x16{};
    st.m = -kUnseenBase;
    st.lr = st.lu = 0.f;

    // Key tiles the workgroup's rows can see (as in the main kernel).
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
    const uint32_t kv_bytes = (uint32_t)klen * D * 2;

    Ctx cx;
    cx.wk = rsrc_words(p.k, slice * 2, kv_bytes);
    cx.wv = rsrc_words(p.v, slice * 2, kv_bytes);
    cx.lds = lds;
    {
      const int row = lane & 31;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) cx.koff[ks] = row * ROWB + (kslot<128>(row, 2 * (pw * KS + ks) + half) << 4);
      const int g = lane >> 4;
      const int key = 4 * (g >> 1) + ((lane >> 2) & 3);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const int dim = 32 * (pw * VB + vb) + 16 * (g & 1) + 4 * (lane & 3);
        cx.voff[vb] = key * ROWB + (((dim >> 3) ^ swz_v<128>(key)) << 4) + ((dim & 7) << 1);
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + THREADS * i;
        const int r = c / (ROWB / 16), col = c % (ROWB / 16);
        cx.gdk[i] = (r * D + klog<128>(r, col) * 8) * 2;
        cx.gdv[i] = (r * D + (col ^ swz_v<128>(r)) * 8) * 2;
      }
      cx.dma = __builtin_amdgcn_readfirstlane((tid & ~63) * 16);
    }
    cx.tfirst = tfirst;
    cx.qw0 = qw0;
    cx.n = klen;
    cx.wl = wl;
    cx.wr = wr;
    cx.lane = lane;
    cx.c2 = p.scale_log2;
    lds_char* xch = lds + RING * SLOTB;

    prologue_loads<0>(cx);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((PF - 1) * CPT) : "memory");
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) steps<0>(cx, st, t, xch);
    // Loads issued ahead past the last tile: let them land before the
    // workgroup's LDS is released.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue: O / l, stores; LSE from the pair's first wave.  As in the
    // main kernel, the rows go out through LDS (the ring is free once every
    // wave has passed the barrier below) as 16-byte pieces of whole runs of
    // the row instead of 8-byte pieces of 32 rows: each wave stages half of
    // its output blocks at a time in a 16 KiB region of its own (32 rows x
    // OB/2 blocks x 64 bytes, chunks at chunk ^ (row mod 16)).  Measured
    // against the direct stores: +1% to +4% at d = 512 and 1024.
    settle_o(st);
    float lo, hi;
    halves(st.lr, lo, hi);
    const float l_tot = lo + hi;
    const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    __syncthreads();
    constexpr int HB = OB / 2;            // output blocks per half
    constexpr int RB = HB * 64;           // staged bytes per row
    static_assert(NW * 32 * RB <= RING * SLOTB, "output staging fits the ring");
    lds_char* ob_lds = lds + wave * 32 * RB;
    const int srow = lane & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < HB; ++i) {
        const int ob = h * HB + i;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack2<BF16>(st.o[ob][4 * g + 0] * inv, st.o[ob][4 * g + 1] * inv);
          w[1] = pack2<BF16>(st.o[ob][4 * g + 2] * inv, st.o[ob][4 * g + 3] * inv);
          // dims 8 g + 4 half .. +3 of block ob: chunk 4 i + g, second half of it for half = 1
          *(__attribute__((address_space(3))) u32x2*)(ob_lds + srow * RB + (((4 * i + g) ^ (srow & 15)) << 4) +
                                                       8 * half) = w;
        }
      }
#pragma unroll
      for (int it = 0; it < 32 * HB * 4 / 64; ++it) {
        const int c = it * 64 + lane;
        const int row = c / (HB * 4), col = c % (HB * 4);
        const int ob = h * HB + col / 4;
        const int dim = (ob / VB) * CW + 32 * (pw * VB + ob % VB) + 8 * (col % 4);
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(ob_lds + row * RB + ((col ^ (row & 15)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, ((qw0 + row) * D + dim) * 2, 0, 0);
      }
    }
    float l_lse = l_tot;
    if constexpr (LSE_FP32) {
      halves(st.lu, lo, hi);
      l_lse = lo + hi;
    }
    if (pw == 0 && half == 0) {
      const float lse = (l_lse > 0.f) ? (st.m + __builtin_amdgcn_logf(l_lse)) * 0.69314718055994531f
                                      : __builtin_inff();
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qrow * 4, 0, 0);
    }
  }
};

template <int D, bool BF16, int MASK>
__global__ void __launch_bounds__((Fa2Wide<D, BF16, MASK>::THREADS), 1) fa2_wide_kernel(const Params p) {
  extern __shared__ __attribute__((aligned(16))) char lds_generic[];
  Fa2Wide<D, BF16, MASK>::run(
      p, (__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)lds_generic);
}

}  // namespace fa2
