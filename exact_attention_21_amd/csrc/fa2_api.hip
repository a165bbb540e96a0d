// C ABI of the FlashAttention-2 forward library (declared in include/fa2.h).
//
// Host side only: argument validation, tile-configuration choice, grid
// mapping and the launch.  Every check runs before the first HIP call, so a
// rejected call enqueues nothing.
#include "fa2.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <unordered_map>

#include "fa2_bwd.hpp"
#include "fa2_kernel.hpp"
#include "fa2_wide.hpp"

// Head dims compiled into the library: a bit mask (bit 0: d = 32, then 64, 96,
// 128, 256, 512, 1024), all of them unless FA2_DIMS says otherwise.  Builds of
// the library with a design switch flipped, made to measure that switch,
// compile only the head dims they are measured on; a head dim left out is
// rejected as unsupported.
#ifndef FA2_DIMS
#define FA2_DIMS 0x7f
#endif

namespace {

constexpr bool built_d(int64_t d) {
  return (FA2_DIMS >> (d == 32 ? 0 : d == 64 ? 1 : d == 96 ? 2 : d == 128 ? 3 : d == 256 ? 4 : d == 512 ? 5 : 6)) & 1;
}

// Tile configuration per head dimension: keys per K/V tile, waves per
// workgroup, 32-row query blocks per wave, split-KV wave groups (2: two
// groups of 4 waves over the same rows).
struct TileCfg {
  int bc;
  int nw;
  int qb;
  int kvg;
};

// Two waves per SIMD let one wave's softmax issue beside the other's MFMAs.
// d = 32, 64 and 128 have two forms.  The 8-wave form runs one workgroup per
// CU (two waves per SIMD): at d = 32 and 64 in two split-KV groups of 4
// waves, at d = 128 as 8 waves of 32 rows on one K/V stream, except without
// a mask, where 4 waves of 64 rows (two query blocks per wave, one wave per
// SIMD, the same 256 rows) share each K/V fragment between two blocks:
// +2% to +3% on unmasked grids of one and two rounds, -1% to +0.4% causal,
// -1.4% on the padded batch (same-process A/B).  The 4-wave form runs two workgroups
// per CU on one K/V stream each, which hide each other's prologue and
// epilogue (choose_eight picks by grid size).  At d = 32 and 64 both forms
// cover the same rows; the 4-wave form of d = 128 covers 128 rows instead of
// 256.  d = 32 and 96 use 64-key tiles: with 32 keys their tiles have fewer
// 16-byte chunks than the threads that load them (d = 32) or a fractional
// number per thread (d = 96).  d = 96 runs without split-KV so that its ring
// (96 KiB) fits the LDS.
constexpr bool has_two_forms(int64_t d) { return d == 32 || d == 64 || d == 128; }

constexpr TileCfg cfg_for(int64_t d, bool eight = true, bool unmasked = false) {
  return d == 32    ? (eight ? TileCfg{64, 8, 1, 2} : TileCfg{64, 4, 1, 1})
         : d == 64  ? (eight ? TileCfg{32, 8, 2, 2} : TileCfg{32, 4, 2, 1})
         : d == 96  ? TileCfg{64, 4, 1, 1}
         : d == 128 ? (eight ? (unmasked ? TileCfg{32, 4, 2, 1} : TileCfg{32, 8, 1, 1}) : TileCfg{32, 4, 1, 1})
                    : TileCfg{32, 4, 1, 1};
}

template <int D, bool EIGHT = true>
using KernelFor = fa2::Fa2Fwd<D, cfg_for(D, EIGHT).bc, cfg_for(D, EIGHT).nw, cfg_for(D, EIGHT).qb,
                              cfg_for(D, EIGHT).kvg, false, false>;
static_assert(KernelFor<32, false>::BR == KernelFor<32>::BR && KernelFor<64, false>::BR == KernelFor<64>::BR,
              "both forms of d = 32 and 64 cover the same rows");
// The unmasked 8-wave-grid form of d = 128 covers the rows, and takes the
// LDS, of the 8-wave form.
using KernelFor128Unmasked = fa2::Fa2Fwd<128, cfg_for(128, true, true).bc, cfg_for(128, true, true).nw,
                                         cfg_for(128, true, true).qb, cfg_for(128, true, true).kvg, false, false>;
static_assert(KernelFor128Unmasked::BR == KernelFor<128>::BR &&
                  KernelFor128Unmasked::LDS_BYTES == KernelFor<128>::LDS_BYTES,
              "both forms of the d = 128 8-wave grid cover the same rows in the same LDS");
// Head dims 512 and 1024 run the chunked kernel (fa2_wide.hpp).
template <int D>
using WideFor = fa2::Fa2Wide<D, false, fa2::kMaskNone>;

// Query rows per workgroup; `eight` selects the form where there are two.
constexpr int rows_per_wg(int64_t d, bool eight = true) {
  return d == 32 ? KernelFor<32>::BR : d == 64 ? KernelFor<64>::BR : d == 96 ? KernelFor<96>::BR
         : d == 128 ? (eight ? KernelFor<128>::BR : KernelFor<128, false>::BR) : d == 256 ? KernelFor<256>::BR
         : d == 512 ? WideFor<512>::BR : WideFor<1024>::BR;
}

constexpr int lds_bytes_for(int64_t d, bool eight = true) {
  return d == 32 ? (eight ? KernelFor<32>::LDS_BYTES : KernelFor<32, false>::LDS_BYTES)
         : d == 64 ? (eight ? KernelFor<64>::LDS_BYTES : KernelFor<64, false>::LDS_BYTES)
         : d == 96 ? KernelFor<96>::LDS_BYTES
         : d == 128 ? (eight ? KernelFor<128>::LDS_BYTES : KernelFor<128, false>::LDS_BYTES)
         : d == 256 ? KernelFor<256>::LDS_BYTES : d == 512 ? WideFor<512>::LDS_BYTES : WideFor<1024>::LDS_BYTES;
}

constexpr int threads_for(int64_t d, bool eight = true, bool unmasked = false) {
  return d == 512 ? WideFor<512>::THREADS : d == 1024 ? WideFor<1024>::THREADS : cfg_for(d, eight, unmasked).nw * 64;
}

// Compute units of the current device (256, MI355X's count, when no device
// can be queried), looked up once per device.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev] = n;
  return n;
}

// The 8-wave form (see cfg_for) unless the grid gives every CU enough
// workgroups of the 4-wave form.  `grid` is the grid of the 8-wave form.
// Measured, same-process A/B of the two forms:
//   d = 32 and 64, no mask: split-KV +1% to +2% at one workgroup per CU,
//     even at two, the 4-wave form +2% to +4% beyond and +35% at N = 512
//     (d = 64);
//   causal, fp16 d = 64: split-KV +11% at two per CU (the query tiles differ
//     in length, and two per CU balance only over several rounds), the 4-wave
//     form +3% to +13% from three;
//   bf16 d = 64 under any mask: the 4-wave form +11% to +32% at every grid
//     tried (one to five per CU): the split-KV form's 8 waves spill there;
//   windows (fp16 d = 64) and d = 32 under a mask: the 4-wave form +4% to
//     +23% at two per CU, even at three;
//   d = 128 (8-wave grid in workgroups per CU): no mask, the 4-wave form +27%
//     at 0.5, -6% at 1 (three shapes) and -5% at 2; causal, +16% to +38% at
//     0.5 and 1 (four shapes), -1% at 1.5, -6% at 2.  The general mask keeps
//     the 8-wave form (not measured).  (Without a mask the 8-wave choice runs
//     the 64-row-wave form, see cfg_for; these figures predate it.)
bool choose_eight(int64_t d, int64_t grid, int mask, int dtype) {
  if (!has_two_forms(d)) return true;
  if (d == 128) {
    if (mask == fa2::kMaskGeneral) return true;
    return mask == fa2::kMaskCausal ? grid > device_cus() : grid >= device_cus();
  }
  if (!FA2_SPLIT_KV) return false;
  if (mask != fa2::kMaskNone && d == 64 && dtype == FA2_DTYPE_BF16) return false;
  const int64_t per_cu = (mask == fa2::kMaskCausal && d == 64) ? 3 : 2;
  return grid < per_cu * device_cus();
}

// XCDs of a gfx950 device (32 compute units each); the dispatcher deals
// workgroups to them round robin by index.
constexpr int kXcds = 8;

// Slices per group of the work order (fa2::work_item): a multiple of the XCD
// count whose query tiles fill FA2_XCD_GROUPS rounds of one XCD's resident
// workgroups, so an XCD walks the keys of few slices at a time and reads each
// K/V tile from HBM about once; all slices when that is no fewer.
//
// Under a mask that makes query tiles differ in length (causal, key lengths,
// a one-sided window) the plain order (longest query tiles first over all
// slices) balances the CUs, and groups trade some of that balance for L2
// reuse; they pay only where the plain order runs at most 2 query tiles of a
// slice at once on an XCD (resident x XCDs <= 2 x slices).  Measured, groups against the
// plain order: padded causal d = 128 with 128 slices +12% to +15%, causal
// d = 64 to 128 with 128 to 512 slices +2% to +7%, no mask +3% to +18% (the
// most at N = 512, d = 256); causal with 32 or 64 slices (4 to 8 query tiles
// of a slice at once) -1% to -4%, which the plain order keeps.
int slice_group(const fa2::Params& p, int wgs_per_cu, int mask) {
  const int bh = p.bh;
  if (FA2_XCD_GROUPS <= 0) return bh;
  const int64_t resident = (int64_t)std::max(1, device_cus() / kXcds) * std::max(1, wgs_per_cu);
  // A window bounded on both sides without key lengths gives every query tile
  // but the first few the same work, as no mask does (measured 0% to +3%
  // from groups on windows of 16 to 64 heads).
  const bool even = mask == fa2::kMaskNone ||
                    (mask == fa2::kMaskGeneral && !p.key_lens && p.wl != fa2::kNoBound && p.wr != fa2::kNoBound);
  if (!even && kXcds * resident > 2 * (int64_t)bh) return bh;
  const int64_t group = kXcds * std::max<int64_t>(1, FA2_XCD_GROUPS * resident / p.n_qtiles);
  return group >= bh ? bh : (int)group;
}

// Rows past N that a launch may address (see check_shape).
constexpr int64_t kPadRows = 256;
static_assert(KernelFor<32>::BR <= kPadRows && KernelFor<64>::BR <= kPadRows && KernelFor<96>::BR <= kPadRows &&
                  KernelFor<128>::BR <= kPadRows && KernelFor<256>::BR <= kPadRows &&
                  WideFor<512>::BR <= kPadRows && WideFor<1024>::BR <= kPadRows,
              "query tile padding");
// The chunked kernel loads one key tile past its range.
static_assert(WideFor<512>::BC <= kPadRows && WideFor<1024>::BC <= kPadRows, "key tile padding (chunked)");
static_assert(4 * cfg_for(32).bc <= kPadRows && 4 * cfg_for(64).bc <= kPadRows && 4 * cfg_for(96).bc <= kPadRows &&
                  4 * cfg_for(128).bc <= kPadRows && 4 * cfg_for(256).bc <= kPadRows,
              "key tile padding");

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

fa2_status_t check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int64_t* grid) {
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_UNSUPPORTED_DTYPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256 && d != 512 && d != 1024)
    return FA2_ERR_UNSUPPORTED_HEAD_DIM;
  if (!built_d(d)) return FA2_ERR_UNSUPPORTED_HEAD_DIM;
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_BAD_SHAPE;
  const int64_t br = rows_per_wg(d);
  // One head's slice is addressed with signed 32-bit byte offsets, including
  // the rows past N that a workgroup touches: the rest of the last query tile
  // (fewer than R <= 256 rows) and the fully masked key tiles that round a
  // split-KV range up (fewer than 4 tiles of at most 64 keys).
  if ((N + kPadRows) * d * 2 >= (int64_t(1) << 31)) return FA2_ERR_BAD_SHAPE;
  if (B > (int64_t(1) << 31) / H) return FA2_ERR_BAD_SHAPE;
  const int64_t bh = B * H;
  const int64_t tiles = (N + br - 1) / br;
  if (tiles > ((int64_t(1) << 31) - 1) / bh) return FA2_ERR_BAD_SHAPE;
  if (grid) *grid = tiles * bh;
  return FA2_OK;
}

// Workgroups of a kernel that one compute unit holds at once (registers and
// LDS), 1 when the runtime cannot say.
int resident_per_cu(const void* kern, int threads, int lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds) != hipSuccess || n < 1) return 1;
  return n;
}

// Per-device set-up of one kernel: its dynamic LDS limit raised to `lds`
// bytes and its resident workgroups per CU, done once for each device the
// kernel is launched on (each template instantiation has its own cache).
struct KernelSetup {
  hipError_t err;
  int per_cu;
};
template <typename Tag>
KernelSetup kernel_setup(const void* kern, int threads, int lds) {
  static std::mutex mu;
  static std::unordered_map<int, KernelSetup> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  KernelSetup k{hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds), 1};
  if (k.err == hipSuccess) k.per_cu = resident_per_cu(kern, threads, lds);
  cache[dev] = k;
  return k;
}

template <int D, int BC, int NW, int QB, int KVG, bool BF16, int MASK>
hipError_t launch(const fa2::Params& p, int64_t grid, hipStream_t stream) {
  constexpr int lds = fa2::Fa2Fwd<D, BC, NW, QB, KVG, BF16, MASK>::LDS_BYTES;
  static_assert(lds == lds_bytes_for(D, true) || lds == lds_bytes_for(D, false), "LDS size");
  auto kern = fa2::fa2_fwd_kernel<D, BC, NW, QB, KVG, BF16, MASK>;
  const KernelSetup k = kernel_setup<fa2::Fa2Fwd<D, BC, NW, QB, KVG, BF16, MASK>>((const void*)kern, NW * 64, lds);
  if (k.err != hipSuccess) return k.err;
  fa2::Params q = p;
  q.group = slice_group(p, k.per_cu, MASK);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds, stream, q);
  return hipGetLastError();
}

template <int D, bool BF16, int MASK>
hipError_t launch_wide(const fa2::Params& p, int64_t grid, hipStream_t stream) {
  using W = fa2::Fa2Wide<D, BF16, MASK>;
  static_assert(W::LDS_BYTES == lds_bytes_for(D) && W::BR == rows_per_wg(D), "chunked kernel shape");
  auto kern = fa2::fa2_wide_kernel<D, BF16, MASK>;
  const KernelSetup k = kernel_setup<W>((const void*)kern, W::THREADS, W::LDS_BYTES);
  if (k.err != hipSuccess) return k.err;
  fa2::Params q = p;
  q.group = slice_group(p, k.per_cu, MASK);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(W::THREADS), W::LDS_BYTES, stream, q);
  return hipGetLastError();
}

template <int D, bool BF16, int MASK>
hipError_t launch_d(const fa2::Params& p, int64_t grid, hipStream_t stream, bool eight) {
  if constexpr (!built_d(D)) {
    return hipErrorInvalidValue;  // not reached: check_shape rejects it
  } else if constexpr (D >= 512) {
    return launch_wide<D, BF16, MASK>(p, grid, stream);
  } else if constexpr (has_two_forms(D)) {
    constexpr TileCfg s = cfg_for(D, true, MASK == fa2::kMaskNone), u = cfg_for(D, false);
    return eight ? launch<D, s.bc, s.nw, s.qb, s.kvg, BF16, MASK>(p, grid, stream)
                 : launch<D, u.bc, u.nw, u.qb, u.kvg, BF16, MASK>(p, grid, stream);
  } else {
    constexpr TileCfg c = cfg_for(D);
    return launch<D, c.bc, c.nw, c.qb, c.kvg, BF16, MASK>(p, grid, stream);
  }
}

template <bool BF16, int MASK>
hipError_t launch_dt(int64_t d, const fa2::Params& p, int64_t grid, hipStream_t stream, bool eight) {
  switch (d) {
    case 32: return launch_d<32, BF16, MASK>(p, grid, stream, eight);
    case 64: return launch_d<64, BF16, MASK>(p, grid, stream, eight);
    case 96: return launch_d<96, BF16, MASK>(p, grid, stream, eight);
    case 128: return launch_d<128, BF16, MASK>(p, grid, stream, eight);
    case 256: return launch_d<256, BF16, MASK>(p, grid, stream, eight);
    case 512: return launch_d<512, BF16, MASK>(p, grid, stream, eight);
    default: return launch_d<1024, BF16, MASK>(p, grid, stream, eight);
  }
}

template <bool BF16>
hipError_t launch_mask(int mask, int64_t d, const fa2::Params& p, int64_t grid, hipStream_t stream, bool eight) {
  switch (mask) {
    case fa2::kMaskNone: return launch_dt<BF16, fa2::kMaskNone>(d, p, grid, stream, eight);
    case fa2::kMaskCausal: return launch_dt<BF16, fa2::kMaskCausal>(d, p, grid, stream, eight);
    default: return launch_dt<BF16, fa2::kMaskGeneral>(d, p, grid, stream, eight);
  }
}

// Checks shared by both entry points (everything but the mask arguments),
// then the launch.  key_lens (general mask only) may be null.
fa2_status_t checked_launch(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
                            int64_t H, int64_t N, int64_t d, float scale, int mask, int64_t wl, int64_t wr,
                            const int32_t* key_lens, int dtype, void* stream) {
  if (!Q || !K || !V || !O || !LSE) return FA2_ERR_NULL_POINTER;
  int64_t grid = 0;
  const fa2_status_t st = check_shape(B, H, N, d, dtype, &grid);
  if (st != FA2_OK) return st;
  if (!std::isfinite(scale)) return FA2_ERR_BAD_SCALE;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return FA2_ERR_MISALIGNED;
  if (((uintptr_t)LSE | (uintptr_t)key_lens) & 3u) return FA2_ERR_MISALIGNED;
  const size_t tensor_bytes = (size_t)(B * H * N * d) * 2;
  const size_t lse_bytes = (size_t)(B * H * N) * 4;
  const size_t len_bytes = key_lens ? (size_t)B * 4 : 0;
  if (overlaps(O, tensor_bytes, Q, tensor_bytes) || overlaps(O, tensor_bytes, K, tensor_bytes) ||
      overlaps(O, tensor_bytes, V, tensor_bytes) || overlaps(LSE, lse_bytes, Q, tensor_bytes) ||
      overlaps(LSE, lse_bytes, K, tensor_bytes) || overlaps(LSE, lse_bytes, V, tensor_bytes) ||
      overlaps(LSE, lse_bytes, O, tensor_bytes) || overlaps(O, tensor_bytes, key_lens, len_bytes) ||
      overlaps(LSE, lse_bytes, key_lens, len_bytes))
    return FA2_ERR_OVERLAP;

  // The form, chosen on the 8-wave form's grid; the 4-wave form of d = 128
  // covers fewer rows per workgroup, so its grid is recomputed.
  const bool eight = choose_eight(d, grid, mask, dtype);
  const int br = rows_per_wg(d, eight);
  grid = (N + br - 1) / br * (B * H);
  fa2::Params p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.n = (int)N;
  p.bh = (int)(B * H);
  p.n_qtiles = (int)((N + br - 1) / br);
  p.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
  p.q_sign = std::signbit(scale) && scale != 0.f ? 0x80008000u : 0u;
  // A bound of N or more hides nothing (N < kNoBound by the size limits).
  p.wl = (wl < 0 || wl >= N) ? fa2::kNoBound : (int)wl;
  p.wr = (wr < 0 || wr >= N) ? fa2::kNoBound : (int)wr;
  p.key_lens = key_lens;
  p.heads = (int)H;
  p.group = p.bh;  // set per kernel at launch (slice_group)

  hipStream_t s = (hipStream_t)stream;
  const hipError_t err = dtype == FA2_DTYPE_BF16 ? launch_mask<true>(mask, d, p, grid, s, eight)
                                                 : launch_mask<false>(mask, d, p, grid, s, eight);
  return err == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

// ---- backward ----------------------------------------------------------
// Slices per group of the backward work order (fa2::bwd_work_item): 8 (one
// per XCD) times the number of a slice's tiles that fill one round of an
// XCD's resident workgroups, at least 8; all slices when that is no fewer.
// Groups are taken under a mask with 128 slices or more (16 per XCD); the
// plain order (heads fastest over all slices, the longest tiles of every
// slice first) otherwise.  Measured, same-process A/B against the plain
// order: masked with 128 to 256 slices +1% to +6% (padded causal d = 128
// +5.7%, causal B8 H16 N4096 d = 128 +5.5%); causal with 32 slices -2% to
// -3%; no mask with 128 slices -2% (d = 128) to +2% (d = 64); 4 or 8
// slices unchanged.
#ifndef FA2_BWD_GROUPS
#define FA2_BWD_GROUPS 1
#endif
int bwd_slice_group(int bh, int n_tiles, int wgs_per_cu, int mask) {
  if (!FA2_BWD_GROUPS || mask == fa2::kMaskNone || bh < 16 * kXcds) return bh;
  const int64_t resident = (int64_t)std::max(1, device_cus() / kXcds) * std::max(1, wgs_per_cu);
  const int64_t group = kXcds * std::max<int64_t>(1, resident / std::max(1, n_tiles));
  return group >= bh ? bh : (int)group;
}

// Steps per phase of the backward work order (fa2::bwd_work_item): two
// phases when the slices are grouped and carry key lengths, whose work then
// differs from slice to slice, so that the grouped order's last groups do not
// start their long tiles at the end of the launch; one phase otherwise.
// Measured, same-process A/B: padded causal d = 128 (128 slices) +7.8%;
// plain causal grids of 128 and 256 slices, where every group has the same
// work, -1.3% to +0.7%, which one phase keeps.
int bwd_phase_tiles(int n_tiles, int group, int bh, const int* key_lens) {
  return key_lens && group < bh ? (n_tiles + 1) / 2 : n_tiles;
}

// Waves per workgroup of the two backward kernels (32 rows each).
constexpr int kBwdWaves = 4;

template <int D, bool BF16, int MASK>
hipError_t launch_bwd(const fa2::BwdParams& base, hipStream_t stream) {
  using KQ = fa2::Fa2BwdQ<D, kBwdWaves, BF16, MASK>;
  using KKV = fa2::Fa2BwdKV<D, kBwdWaves, BF16, MASK>;
  auto kq = fa2::fa2_bwd_q_kernel<D, kBwdWaves, BF16, MASK>;
  auto kkv = fa2::fa2_bwd_kv_kernel<D, kBwdWaves, BF16, MASK>;
  const KernelSetup sq = kernel_setup<KQ>((const void*)kq, KQ::THREADS, KQ::LDS_BYTES);
  if (sq.err != hipSuccess) return sq.err;
  const KernelSetup skv = kernel_setup<KKV>((const void*)kkv, KKV::THREADS, KKV::LDS_BYTES);
  if (skv.err != hipSuccess) return skv.err;
  // dQ and Delta first: the dK/dV kernel reads Delta.
  fa2::BwdParams p = base;
  p.n_tiles = (p.n + KQ::BQ - 1) / KQ::BQ;
  p.group = bwd_slice_group(p.bh, p.n_tiles, sq.per_cu, MASK);
  p.phase_tiles = bwd_phase_tiles(p.n_tiles, p.group, p.bh, p.key_lens);
  hipLaunchKernelGGL(kq, dim3((unsigned)((int64_t)p.n_tiles * p.bh)), dim3(KQ::THREADS), KQ::LDS_BYTES, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  p.n_tiles = (p.n + KKV::BK - 1) / KKV::BK;
  p.group = bwd_slice_group(p.bh, p.n_tiles, skv.per_cu, MASK);
  p.phase_tiles = bwd_phase_tiles(p.n_tiles, p.group, p.bh, p.key_lens);
  hipLaunchKernelGGL(kkv, dim3((unsigned)((int64_t)p.n_tiles * p.bh)), dim3(KKV::THREADS), KKV::LDS_BYTES, stream,
                     p);
  return hipGetLastError();
}

template <bool BF16, int MASK>
hipError_t launch_bwd_d(int64_t d, const fa2::BwdParams& p, hipStream_t stream) {
  return d == 32    ? launch_bwd<32, BF16, MASK>(p, stream)
         : d == 64  ? launch_bwd<64, BF16, MASK>(p, stream)
         : d == 96  ? launch_bwd<96, BF16, MASK>(p, stream)
         : d == 128 ? launch_bwd<128, BF16, MASK>(p, stream)
                    : launch_bwd<256, BF16, MASK>(p, stream);
}

template <bool BF16>
hipError_t launch_bwd_mask(int mask, int64_t d, const fa2::BwdParams& p, hipStream_t stream) {
  switch (mask) {
    case fa2::kMaskNone: return launch_bwd_d<BF16, fa2::kMaskNone>(d, p, stream);
    case fa2::kMaskCausal: return launch_bwd_d<BF16, fa2::kMaskCausal>(d, p, stream);
    default: return launch_bwd_d<BF16, fa2::kMaskGeneral>(d, p, stream);
  }
}

// Rows per workgroup of either backward kernel (the grid-size limit).
constexpr int64_t kBwdRows = 32 * kBwdWaves;
static_assert(fa2::Fa2BwdQ<64, kBwdWaves, false, 0>::BQ == kBwdRows &&
                  fa2::Fa2BwdKV<64, kBwdWaves, false, 0>::BK == kBwdRows,
              "backward tiles");
static_assert(kBwdRows <= kPadRows && fa2::Fa2BwdQ<64, kBwdWaves, false, 0>::BC <= kPadRows &&
                  fa2::Fa2BwdKV<64, kBwdWaves, false, 0>::BQ <= kPadRows,
              "backward rows past N stay within the padded slice");

fa2_status_t bwd_check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_UNSUPPORTED_DTYPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA2_ERR_UNSUPPORTED_HEAD_DIM;
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_BAD_SHAPE;
  if ((N + kPadRows) * d * 2 >= (int64_t(1) << 31)) return FA2_ERR_BAD_SHAPE;
  if (B > (int64_t(1) << 31) / H) return FA2_ERR_BAD_SHAPE;
  const int64_t tiles = (N + kBwdRows - 1) / kBwdRows;
  if (tiles > ((int64_t(1) << 31) - 1) / (B * H)) return FA2_ERR_BAD_SHAPE;
  return FA2_OK;
}

// Workspace of fa2_bwd_noalloc: one array per device, in the library's code
// object, for callers that cannot allocate.  Host code never uses the
// array's own name as a device address: the address is looked up once per
// device (scratch_workspace) and that pointer is what the kernels get.
constexpr int64_t kScratchFloats = int64_t(1) << 22;  // 16 MiB: B * H * N <= 2^21
static __device__ __align__(256) float scratch[kScratchFloats];

// The device address of `scratch` on the current device (looked up on the
// first call on each device), or null with *err set.
float* scratch_workspace(int64_t floats, fa2_status_t* err) {
  if (floats > kScratchFloats) {
    *err = FA2_ERR_TOO_LARGE;
    return nullptr;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = FA2_ERR_HIP;
    return nullptr;
  }
  static std::mutex mu;
  static std::unordered_map<int, float*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it != ptrs.end()) return it->second;
  float* ptr = nullptr;
  if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    *err = FA2_ERR_HIP;
    return nullptr;
  }
  ptrs[dev] = ptr;
  return ptr;
}

// Checks and launch of both backward entry points.  `get_scratch` (the
// allocation-free entry point) supplies the workspace after every argument
// check has passed; otherwise `workspace` is the caller's.
fa2_status_t bwd_checked_launch(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                const float* LSE, void* dQ, void* dK, void* dV, float* workspace, int64_t B,
                                int64_t H, int64_t N, int64_t d, float scale, int mask, int64_t wl, int64_t wr,
                                const int32_t* key_lens, int dtype, void* stream,
                                float* (*get_scratch)(int64_t, fa2_status_t*)) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA2_ERR_NULL_POINTER;
  const fa2_status_t st = bwd_check_shape(B, H, N, d, dtype);
  if (st != FA2_OK) return st;
  if (!std::isfinite(scale)) return FA2_ERR_BAD_SCALE;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)dO | (uintptr_t)dQ | (uintptr_t)dK |
       (uintptr_t)dV) & 15u)
    return FA2_ERR_MISALIGNED;
  if (((uintptr_t)LSE | (uintptr_t)workspace | (uintptr_t)key_lens) & 3u) return FA2_ERR_MISALIGNED;
  const size_t tb = (size_t)(B * H * N * d) * 2;
  const size_t rb = (size_t)(B * H * N) * 4;
  const void* ins[7] = {Q, K, V, O, dO, LSE, key_lens};
  const size_t in_bytes[7] = {tb, tb, tb, tb, tb, rb, key_lens ? (size_t)B * 4 : 0};
  const void* outs[4] = {dQ, dK, dV, workspace};
  const size_t out_bytes[4] = {tb, tb, tb, workspace ? 2 * rb : 0};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA2_ERR_OVERLAP;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA2_ERR_OVERLAP;
  }
  if (get_scratch) {
    fa2_status_t err = FA2_OK;
    workspace = get_scratch(2 * B * H * N, &err);
    if (!workspace) return err;
  }
  fa2::BwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.dout = dO;
  p.lse = LSE;
  p.delta = workspace;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  p.n = (int)N;
  p.bh = (int)(B * H);
  p.n_tiles = 0;  // set per kernel
  p.scale = scale;
  p.c2 = scale * 1.4426950408889634f;
  // A bound of N or more hides nothing (N < kNoBound by the size limits).
  p.wl = (wl < 0 || wl >= N) ? fa2::kNoBound : (int)wl;
  p.wr = (wr < 0 || wr >= N) ? fa2::kNoBound : (int)wr;
  p.key_lens = key_lens;
  p.heads = (int)H;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t err = dtype == FA2_DTYPE_BF16 ? launch_bwd_mask<true>(mask, d, p, s)
                                                 : launch_bwd_mask<false>(mask, d, p, s);
  return err == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

}  // namespace

extern "C" {

const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL_POINTER: return "a buffer pointer is NULL";
    case FA2_ERR_BAD_SHAPE: return "bad shape: B, H, N must be >= 1 and within the size limits";
    case FA2_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dimension (supported: 32, 64, 96, 128, 256, 512, 1024)";
    case FA2_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype (supported: fp16, bf16)";
    case FA2_ERR_BAD_SCALE: return "scale is not a finite number";
    case FA2_ERR_MISALIGNED:
      return "a [B, H, N, d] tensor is not 16-byte aligned, or LSE, key_lens or the workspace not 4-byte aligned";
    case FA2_ERR_OVERLAP: return "an output overlaps an input or another output";
    case FA2_ERR_HIP: return "the HIP runtime reported an error at launch";
    case FA2_ERR_TOO_LARGE: return "B * H * N exceeds what the allocation-free entry point's scratch holds";
    default: return "unknown status";
  }
}

fa2_status_t fa2_launch_info(int64_t B, int64_t H, int64_t N, int64_t d, int is_causal, int dtype,
                             int64_t* workgroups, int* threads, int* rows_per_wg,
                             int* keys_per_tile, int* lds_bytes) {
  int64_t grid = 0;
  const fa2_status_t st = check_shape(B, H, N, d, dtype, &grid);
  if (st != FA2_OK) return st;
  const bool eight = choose_eight(d, grid, is_causal ? fa2::kMaskCausal : fa2::kMaskNone, dtype);
  const TileCfg c = cfg_for(d, eight, !is_causal);
  grid = (N + ::rows_per_wg(d, eight) - 1) / ::rows_per_wg(d, eight) * (B * H);
  if (workgroups) *workgroups = grid;
  if (threads) *threads = threads_for(d, eight, !is_causal);
  if (rows_per_wg) *rows_per_wg = ::rows_per_wg(d, eight);
  if (keys_per_tile) *keys_per_tile = c.bc;
  if (lds_bytes) *lds_bytes = lds_bytes_for(d, eight);
  return FA2_OK;
}

fa2_status_t fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int is_causal,
                     int dtype, void* stream) {
  return checked_launch(Q, K, V, O, LSE, B, H, N, d, scale, is_causal ? fa2::kMaskCausal : fa2::kMaskNone, -1,
                        is_causal ? 0 : -1, nullptr, dtype, stream);
}

fa2_status_t fa2_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale, int64_t window_left,
                            int64_t window_right, const int32_t* key_lens, int dtype, void* stream) {
  // No window is the unmasked kernel and a window with no left bound and
  // right bound 0 the causal one, with or without key lengths (the same
  // results as the general mask, whose extra work is for windows); anything
  // else runs the general mask.
  const bool no_left = window_left < 0 || window_left >= N;
  const bool no_right = window_right < 0 || window_right >= N;
  int mask = fa2::kMaskGeneral;
  if (no_left && no_right) mask = fa2::kMaskNone;
  if (no_left && window_right == 0) mask = fa2::kMaskCausal;
  return checked_launch(Q, K, V, O, LSE, B, H, N, d, scale, mask, window_left, window_right, key_lens, dtype,
                        stream);
}

fa2_status_t fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                     void* dQ, void* dK, void* dV, float* workspace, int64_t B, int64_t H, int64_t N, int64_t d,
                     float scale, int is_causal, int dtype, void* stream) {
  if (!workspace) return FA2_ERR_NULL_POINTER;
  return bwd_checked_launch(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, N, d, scale,
                            is_causal ? fa2::kMaskCausal : fa2::kMaskNone, -1, is_causal ? 0 : -1, nullptr, dtype,
                            stream, nullptr);
}

fa2_status_t fa2_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV, int64_t B, int64_t H, int64_t N,
                             int64_t d, float scale, int is_causal, int dtype, void* stream) {
  return bwd_checked_launch(Q, K, V, O, dO, LSE, dQ, dK, dV, nullptr, B, H, N, d, scale,
                            is_causal ? fa2::kMaskCausal : fa2::kMaskNone, -1, is_causal ? 0 : -1, nullptr, dtype,
                            stream, &scratch_workspace);
}

fa2_status_t fa2_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                            const float* LSE, void* dQ, void* dK, void* dV, float* workspace, int64_t B, int64_t H,
                            int64_t N, int64_t d, float scale, int64_t window_left, int64_t window_right,
                            const int32_t* key_lens, int dtype, void* stream) {
  if (!workspace) return FA2_ERR_NULL_POINTER;
  // No window and no key lengths run the unmasked kernels, a window with no
  // left bound and right bound 0 (no key lengths) the causal ones; anything
  // else the general mask.
  const bool no_left = window_left < 0 || window_left >= N;
  const bool no_right = window_right < 0 || window_right >= N;
  int mask = fa2::kMaskGeneral;
  if (!key_lens && no_left && no_right) mask = fa2::kMaskNone;
  if (!key_lens && no_left && window_right == 0) mask = fa2::kMaskCausal;
  return bwd_checked_launch(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, N, d, scale, mask, window_left,
                            window_right, key_lens, dtype, stream, nullptr);
}

}  // extern "C"
