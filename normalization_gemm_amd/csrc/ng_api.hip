// libnormgemm C ABI: argument checks, strategy choice and kernel launches.
//
// Every entry point validates its arguments on the host before any HIP call,
// then enqueues on the caller's stream and returns; nothing here allocates,
// frees or synchronizes (except ng_workspace_status, which exists to sync).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <algorithm>
#include <mutex>

#include "../../include/normgemm.h"
#include "ng_gemm_kernel.h"
#include "ng_norm_kernel.h"
#include "ng_fold_kernel.h"

// Scratch of ng_gemm_layernorm_noalloc: the cross-workgroup exchange's
// workspace in static device memory, one copy per device, held until the
// process ends.  Zero when the code object is loaded (static storage).  Host
// code never uses the name as an address: each device's address comes from
// hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

thread_local char g_err[512];

ng_status fail(ng_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

ng_status ok() {
  g_err[0] = '\0';
  return NG_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 24;
// Longest row of A [M, K] (and of B stored [N, K]) that a tile can read: the
// tile addresses its (up to 256) rows from one base through 32-bit buffer
// offsets that must stay inside the buffer range (clamped below 2 GiB), and
// 255 * 2K + 2 * 64 <= 0x7FFFFFF0 holds for every K <= 2^22.
constexpr int64_t kMaxRowK = int64_t(1) << 22;

// Tile configurations.
//   Large: 256x256 macro tile, 8 waves (4 along M x 2 along N) of 64x128, two
//          waves per SIMD so that one issues MFMAs while the other waits
//          (MFMA-bound shapes; measured ahead of 4 waves of 128x128).  With B
//          stored [K, N] the k-tiles are 32 deep in 4 stages (128 KB), which
//          keeps 1.5 k64-steps of transfers in flight instead of one: 1-3 %
//          faster on the large shapes than 2 stages of 64.  With B stored
//          [N, K] 2 stages of 64 stay ahead (the deeper loop spills there).
//   Row128: 128 x 128, 4 waves stacked along M (each owns 32 whole rows, so
//           row statistics need no cross-wave exchange), two LDS stages
//           (75 KB), so that two workgroups share a CU and one's loads overlap
//           the other's epilogue: the N <= 128 shapes are HBM-bound.
//           (Measured on 65536x512x128 against 256 x 128 tiles of 8 waves
//           with three stages, one workgroup per CU: 3 % faster; 128 x 128
//           with three stages, 64 x 128 and 8-wave 128 x 128 were slower, and
//           so were 32-deep k-tiles in 3 or 4 stages and persistent grids of
//           64- or 128-row tiles.)  Each row block of A has one reader, so A
//           is fetched nontemporally (19.1 against 19.8 us on that shape).
//   Row256: 128 x 256, 2x2 waves (128 < N <= 256).
template <bool KN> struct TLargeSel {
  using type = ng::Tile<256, 256, 4, 2, false, 2>;
};
template <> struct TLargeSel<true> {
  using type = ng::Tile<256, 256, 4, 2, true, 4, false, 0, 32>;
};
template <bool KN> using TLarge = typename TLargeSel<KN>::type;
template <bool KN> using TRow128 = ng::Tile<128, 128, 4, 1, KN, 2, false, 0, 64, true>;
template <bool KN> using TRow256 = ng::Tile<128, 256, 2, 2, KN>;
//   Wgrad: the 256x256 tile with A stored [K, M] (the reduction over the
//          forward rows), 32-deep k-tiles in 4 stages, and the normalized A
//          rebuilt on the A (RS 1) or B (RS 2) side, one k-tile ahead in LDS.
//          (Measured on 32768x4096x4096, same board: the plain product 783
//          against 855 us for 2 stages of 64; the rebuilt forms 941-950 us,
//          against 972 us for scaling the A fragments in registers and
//          1030 us for scaling the B k-tile in LDS between its wait and its
//          barrier.)
template <int RS> using TWgrad = ng::Tile<256, 256, 4, 2, true, 4, true, RS, 32>;

ng_status check_gemm(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
               int b_layout) {
  // A and C are empty when M == 0 and may then be NULL.
  if (!B || (M != 0 && (!A || !C)))
    return fail(NG_ERR_INVALID_ARG, "A, B and C must be non-NULL");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16))
    return fail(NG_ERR_INVALID_ARG, "A, B and C must be 16-byte aligned");
  if (M < 0 || N < 1 || K < 1)
    return fail(NG_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1 (got M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(NG_ERR_INVALID_ARG, "M, N, K must be at most 2^24");
  if (b_layout != NG_B_KN && b_layout != NG_B_NK)
    return fail(NG_ERR_INVALID_ARG, "b_layout must be NG_B_KN or NG_B_NK (got %d)", b_layout);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(NG_ERR_UNSUPPORTED, "N and K must be multiples of 8 (got N=%lld K=%lld)",
                (long long)N, (long long)K);
  if (K > kMaxRowK)
    return fail(NG_ERR_UNSUPPORTED, "K must be at most 2^22 (got K=%lld)", (long long)K);
  if ((M * K) >= (int64_t(1) << 31) * 8 || (N * K) >= (int64_t(1) << 31) * 8 ||
      (M * N) >= (int64_t(1) << 31) * 8)
    return fail(NG_ERR_UNSUPPORTED, "a matrix has more than 2^34 elements");
  return NG_OK;
}

ng_status check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(NG_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return NG_OK;
}

ng_status check_vec(const void* p, const char* name, size_t align) {
  if (p && !aligned(p, align))
    return fail(NG_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return NG_OK;
}

ng_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(NG_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Diagnostic options (ng_set_debug_option), process-wide.
//   wait bound of the cross-workgroup waits, in polls of ~1 us (-1: 2^20,
//     about a second);
//   widest row reduced inside one workgroup (-1: 256);
//   tile order of the grids (NG_TILE_ORDER_*);
//   k-tile walk of the cross-workgroup grid (NG_K_WALK_*).
std::atomic<int> g_wait_spins{-1};
std::atomic<int> g_k_walk{NG_K_WALK_AUTO};
std::atomic<int> g_row_local_max{-1};
std::atomic<int> g_tile_order{NG_TILE_ORDER_NATURAL};

int wait_spins() {
  const int v = g_wait_spins.load(std::memory_order_relaxed);
  return v < 0 ? (1 << 20) : v;
}

int64_t row_local_max() {
  const int v = g_row_local_max.load(std::memory_order_relaxed);
  return v < 0 ? 256 : v;
}

// (a, c) of the tile walk t -> (a t + c) mod total for the current tile-order
// option: natural (1, 0); reversed (total - 1, total - 1), i.e. total - 1 - t;
// shuffled: a a prime that does not divide total (so a is coprime to it) and
// an offset of a third of the walk.
void tile_order(int64_t total, int* a, int* c) {
  const int mode = g_tile_order.load(std::memory_order_relaxed);
  *a = 1;
  *c = 0;
  if (total <= 1 || mode == NG_TILE_ORDER_NATURAL) return;
  if (mode == NG_TILE_ORDER_REVERSED) {
    *a = (int)(total - 1);
    *c = (int)(total - 1);
    return;
  }
  static const int64_t primes[] = {15485863, 104729, 7919, 9973};
  for (int64_t q : primes) {
    if (total % q != 0) {
      *a = (int)(q % total);
      break;
    }
  }
  *c = (int)(total / 3);
}

ng::GemmParams make_params(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                           float eps) {
  ng::GemmParams p{};
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.C = (uint16_t*)C;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.eps = eps;
  p.spin_limit = wait_spins();
  p.order_a = 1;
  p.order_c = 0;
  return p;
}

template <class T, int EPI>
ng_status launch_grid(ng::GemmParams p, hipStream_t s, const char* what) {
  p.tiles_m = (p.M + T::BM - 1) / T::BM;
  p.tiles_n = (p.N + T::BN - 1) / T::BN;
  const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
  tile_order(grid, &p.order_a, &p.order_c);
  hipLaunchKernelGGL((ng::gemm_kernel<T, EPI>), dim3(grid), dim3(T::NT), 0, s, p);
  return launched(what);
}

// Co-resident workgroups per device for a persistent kernel (cached per
// kernel and device).
ng_status resident_capacity(const void* kernel, int threads, int* cap) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(NG_ERR_HIP, "hipGetDevice failed");
  struct Entry {
    const void* kernel;
    int dev, cap;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int n_cached = 0;
  std::lock_guard<std::mutex> lk(mu);
  for (int i = 0; i < n_cached; ++i) {
    if (cache[i].kernel == kernel && cache[i].dev == dev) {
      *cap = cache[i].cap;
      return NG_OK;
    }
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return fail(NG_ERR_HIP, "occupancy query failed");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(NG_ERR_HIP, "CU count query failed");
  const int c = per_cu * cus;
  if (c <= 0) return fail(NG_ERR_HIP, "persistent kernel cannot be resident");
  if (n_cached < 64) cache[n_cached++] = Entry{kernel, dev, c};
  *cap = c;
  return NG_OK;
}

// Bytes that one round of a persistent grid reads and writes (all of B, the
// round's A panels and its output rows) above which its odd rounds walk the
// k-tiles downwards: past this size the next round's first k-tiles have left
// the 256 MB Infinity Cache when read upwards again.
constexpr uint64_t kWalkBytes = uint64_t(192) << 20;

// rb x cb: row blocks x column tiles (of BM x BN) that one round covers.
bool alternate_walk(const ng::GemmParams& p, int rb, int cb, int BM, int BN,
                    bool several_rounds) {
  const int mode = g_k_walk.load(std::memory_order_relaxed);
  if (!several_rounds) return false;
  if (mode != NG_K_WALK_AUTO) return mode == NG_K_WALK_ALTERNATE;
  const uint64_t rows = std::min<uint64_t>((uint64_t)rb * BM, (uint64_t)p.M);
  const uint64_t cols = std::min<uint64_t>((uint64_t)cb * BN, (uint64_t)p.N);
  const uint64_t round_bytes = 2ull * (cols * p.K + rows * p.K + rows * cols);
  return round_bytes > kWalkBytes;
}

template <class T, int EPI>
ng_status launch_persistent(ng::GemmParams p, hipStream_t s, const char* what) {
  p.tiles_m = (p.M + T::BM - 1) / T::BM;
  p.tiles_n = (p.N + T::BN - 1) / T::BN;
  const long long total = (long long)p.tiles_m * p.tiles_n;
  int cap = 0;
  ng_status st = resident_capacity((const void*)ng::gemm_persistent_kernel<T, EPI>, T::NT, &cap);
  if (st) return st;
  const unsigned grid = (unsigned)(total < cap ? total : cap);
  // the Lazy kernels walk strips of column tiles (one row block each); the
  // tile order permutes the strips
  const long long walked =
      ng::epi_lazy(EPI)
          ? (long long)p.tiles_m * ((p.tiles_n + ng::kLazyStrip - 1) / ng::kLazyStrip)
          : total;
  tile_order(walked, &p.order_a, &p.order_c);
  if constexpr (EPI == ng::EPI_NONE && !T::AKM) {
    // a round: grid tiles, whole rows of tiles where they fit
    const int cb = std::min(p.tiles_n, (int)grid);
    const int rb = std::max(1, std::min(p.tiles_m, (int)grid / cb));
    if (alternate_walk(p, rb, cb, T::BM, T::BN, total > (long long)grid)) {
      int cap2 = 0;
      st = resident_capacity((const void*)ng::gemm_persistent_kernel<T, EPI, true>, T::NT, &cap2);
      if (st) return st;
      hipLaunchKernelGGL((ng::gemm_persistent_kernel<T, EPI, true>),
                         dim3((unsigned)std::min<long long>(grid, cap2)), dim3(T::NT), 0, s, p);
      return launched(what);
    }
  }
  hipLaunchKernelGGL((ng::gemm_persistent_kernel<T, EPI>), dim3(grid), dim3(T::NT), 0, s, p);
  return launched(what);
}

template <class T, bool LN, bool RES, bool BWD = false>
ng_status launch_xwg(ng::GemmParams p, hipStream_t s, const char* what) {
  p.tiles_m = (p.M + T::BM - 1) / T::BM;
  p.tiles_n = (p.N + T::BN - 1) / T::BN;
  int cap = 0;
  ng_status st = resident_capacity((const void*)ng::gemm_xwg_kernel<T, LN, RES, BWD>, T::NT, &cap);
  if (st) return st;
  const int resident = std::min(cap, ng::kXwgMaxResident);
  if (p.tiles_n > resident)
    return fail(NG_ERR_UNSUPPORTED, "row of %d tiles exceeds %d co-resident workgroups",
                p.tiles_n, resident);
  // row blocks per round (the workspace holds one slot per row block of a
  // round, for at most kXwgMaxResident workgroups)
  int R = resident / p.tiles_n;
  if (R > p.tiles_m) R = p.tiles_m;
  p.iters = (p.tiles_m + R - 1) / R;
  const unsigned grid = (unsigned)(R * p.tiles_n);
  tile_order(grid, &p.order_a, &p.order_c);
  // A plain launch: the grid never exceeds what the device holds at once, so
  // on a device not shared with another such grid all workgroups become
  // resident.  (A cooperative launch would guarantee it even then, but was
  // measured to add ~18 us per call.)  Both k-walk variants have the same
  // resources (checked by the occupancy query of each).
  if constexpr (!RES && !BWD) {
    if (alternate_walk(p, R, p.tiles_n, T::BM, T::BN, p.iters > 1)) {
      int cap2 = 0;
      st = resident_capacity((const void*)ng::gemm_xwg_kernel<T, LN, RES, BWD, true>, T::NT,
                             &cap2);
      if (st) return st;
      if (cap2 < (int)grid)
        return fail(NG_ERR_UNSUPPORTED, "alternating k-walk grid of %u workgroups exceeds %d",
                    grid, cap2);
      hipLaunchKernelGGL((ng::gemm_xwg_kernel<T, LN, RES, BWD, true>), dim3(grid), dim3(T::NT),
                         0, s, p);
      return launched(what);
    }
  }
  hipLaunchKernelGGL((ng::gemm_xwg_kernel<T, LN, RES, BWD>), dim3(grid), dim3(T::NT), 0, s, p);
  return launched(what);
}

// Workspace of the cross-workgroup grid: one slot per row block of a round,
// for as many row blocks as a round can hold (at most kXwgMaxResident
// workgroups, and no more than the matrix has), one partial per row and
// column tile.  It does not grow with M past one round.
size_t xwg_bytes(int64_t M, int64_t N) {
  using T = TLarge<true>;
  const int tm = (int)((M + T::BM - 1) / T::BM);
  const int tn = (int)((N + T::BN - 1) / T::BN);
  const int slots = std::max(1, std::min(tm, ng::kXwgMaxResident / tn));
  return ng::XwgLayout::bytes(slots, tn, T::BM);
}

// Strategy choice of the epilogue norms: N <= 128 one 256 x 128 workgroup
// per row block, N <= 256 one 128 x 256 workgroup, wider rows the
// cross-workgroup grid.
template <bool LN, bool RES>
ng_status launch_norm(ng::GemmParams p, bool kn, bool local, hipStream_t s, const char* what) {
  constexpr int EPI = RES ? (LN ? ng::EPI_ROW_LN_RES : ng::EPI_ROW_RMS_RES)
                          : (LN ? ng::EPI_ROW_LN : ng::EPI_ROW_RMS);
  if (local && p.N <= 128)
    return kn ? launch_grid<TRow128<true>, EPI>(p, s, what)
              : launch_grid<TRow128<false>, EPI>(p, s, what);
  if (local)
    return kn ? launch_grid<TRow256<true>, EPI>(p, s, what)
              : launch_grid<TRow256<false>, EPI>(p, s, what);
  return kn ? launch_xwg<TLarge<true>, LN, RES>(p, s, what)
            : launch_xwg<TLarge<false>, LN, RES>(p, s, what);
}

// Shared by ng_gemm_rmsnorm / ng_gemm_layernorm and the residual forms
// (R non-NULL).
// Argument checks of the epilogue norms (everything but the workspace).
ng_status check_gemm_norm(const void* A, const void* B, const void* R, const void* gamma,
                          const void* beta, const void* C, const void* S_out, int64_t M, int64_t N,
                          int64_t K, int b_layout, float eps, const float* mean_out,
                          const float* rstd_out, bool residual) {
  ng_status st = check_gemm(A, B, C, M, N, K, b_layout);
  if (!st) st = check_eps(eps);
  if (!st) st = check_vec(gamma, "gamma", 16);
  if (!st) st = check_vec(beta, "beta", 16);
  if (!st) st = check_vec(mean_out, "mean_out", 4);
  if (!st) st = check_vec(rstd_out, "rstd_out", 4);
  if (st) return st;
  if (residual) {
    if (M != 0 && !R) return fail(NG_ERR_INVALID_ARG, "R must be non-NULL");
    if (!aligned(R, 16) || !aligned(S_out, 16))
      return fail(NG_ERR_INVALID_ARG, "R and S_out must be 16-byte aligned");
    if (S_out && M != 0 && S_out == C)
      return fail(NG_ERR_INVALID_ARG, "S_out and C must be different buffers");
  }
  return NG_OK;
}

ng_status gemm_norm(const void* A, const void* B, const void* R, const void* gamma, const void* beta,
              void* C, void* S_out, int64_t M, int64_t N, int64_t K, int b_layout, float eps,
              float* mean_out, float* rstd_out, void* ws, size_t ws_bytes, hipStream_t s,
              int kind, bool residual, const char* what) {
  ng_status st = check_gemm_norm(A, B, R, gamma, beta, C, S_out, M, N, K, b_layout, eps, mean_out,
                                 rstd_out, residual);
  if (st) return st;
  const bool local = N <= row_local_max();
  if (!local && M > 0) {
    const size_t need = xwg_bytes(M, N);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
      return fail(NG_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed, got %zu",
                  need, ws_bytes);
  }
  if (M == 0) return ok();
  ng::GemmParams p = make_params(A, B, C, M, N, K, eps);
  p.gamma = (const uint16_t*)gamma;
  p.beta = (const uint16_t*)beta;
  p.R = (const uint16_t*)R;
  p.S_out = (uint16_t*)S_out;
  p.mean_out = mean_out;
  p.rstd_out = rstd_out;
  p.ws = (char*)ws;
  p.norm_kind = kind;
  const bool kn = b_layout == NG_B_KN;
  const bool ln = kind == ng::NORM_LAYER;
  if (residual)
    return ln ? launch_norm<true, true>(p, kn, local, s, what)
              : launch_norm<false, true>(p, kn, local, s, what);
  return ln ? launch_norm<true, false>(p, kn, local, s, what)
            : launch_norm<false, false>(p, kn, local, s, what);
}

// Per-device address of `scratch`, taken once per device on the first
// no-allocation call there (with that device current), followed by a zero
// fill on the caller's stream unless the stream is being captured into a
// graph (the array is zero from the load anyway; the fill makes the start
// state explicit without putting a fill into a captured graph).
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
  const char* step = "";
};
ScratchSlot g_scratch_slot[64];

ng_status noalloc_scratch(hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(NG_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(NG_ERR_UNSUPPORTED, "device index %d out of range", dev);
  ScratchSlot& sl = g_scratch_slot[dev];
  std::call_once(sl.once, [&] {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      sl.err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      sl.step = "hipGetSymbolAddress";
      return;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
      (void)hipGetLastError();
      cs = hipStreamCaptureStatusActive;  // unknown: do not enqueue the fill
    }
    if (cs == hipStreamCaptureStatusNone) {
      hipLaunchKernelGGL(ng::fill_zero_kernel, dim3(1024), dim3(256), 0, s, (ng::u32x4*)p,
                         kNoallocScratchBytes / 16, (uint32_t*)nullptr, (size_t)0);
      e = hipGetLastError();
      if (e != hipSuccess) {
        sl.err = e;
        sl.step = "zero fill";
        return;
      }
    }
    sl.ptr = p;
  });
  if (sl.err != hipSuccess)
    return fail(NG_ERR_HIP, "scratch set-up (%s) failed: %s", sl.step, hipGetErrorString(sl.err));
  *out = sl.ptr;
  return NG_OK;
}

}  // namespace

extern "C" {

ng_status ng_gemm_layernorm_noalloc(const ng_bf16* A, const ng_bf16* B, const ng_bf16* gamma,
                                    const ng_bf16* beta, ng_bf16* C, int64_t M, int64_t N,
                                    int64_t K, int b_layout, float eps, float* mean_out,
                                    float* rstd_out, void* stream) {
  ng_status st = check_gemm_norm(A, B, nullptr, gamma, beta, C, nullptr, M, N, K, b_layout, eps,
                                 mean_out, rstd_out, false);
  if (st) return st;
  void* ws = nullptr;
  size_t wsb = 0;
  if (M > 0 && N > row_local_max()) {
    const size_t need = xwg_bytes(M, N);
    if (need > kNoallocScratchBytes)
      return fail(NG_ERR_UNSUPPORTED,
                  "this shape's row exchange needs %zu bytes; the no-allocation variant holds %zu "
                  "(use ng_gemm_layernorm with a workspace)",
                  need, kNoallocScratchBytes);
    st = noalloc_scratch((hipStream_t)stream, &ws);
    if (st) return st;
    wsb = kNoallocScratchBytes;
  }
  return gemm_norm(A, B, nullptr, gamma, beta, C, nullptr, M, N, K, b_layout, eps, mean_out,
                   rstd_out, ws, wsb, (hipStream_t)stream, ng::NORM_LAYER, false,
                   "ng_gemm_layernorm_noalloc");
}

ng_status ng_rmsnorm_gemm_lazy(const ng_bf16* A, const ng_bf16* B, ng_bf16* C, int64_t M, int64_t N,
                         int64_t K, int b_layout, float eps, float* rstd_out, void* stream) {
  ng_status st = check_gemm(A, B, C, M, N, K, b_layout);
  if (!st) st = check_eps(eps);
  if (!st) st = check_vec(rstd_out, "rstd_out", 4);
  if (st) return st;
  if (M == 0) return ok();
  ng::GemmParams p = make_params(A, B, C, M, N, K, eps);
  p.rstd_out = rstd_out;
  hipStream_t s = (hipStream_t)stream;
  const bool kn = b_layout == NG_B_KN;
  if (N <= 128)
    return kn ? launch_grid<TRow128<true>, ng::EPI_LAZY>(p, s, "ng_rmsnorm_gemm_lazy")
              : launch_grid<TRow128<false>, ng::EPI_LAZY>(p, s, "ng_rmsnorm_gemm_lazy");
  return kn ? launch_persistent<TLarge<true>, ng::EPI_LAZY>(p, s, "ng_rmsnorm_gemm_lazy")
            : launch_persistent<TLarge<false>, ng::EPI_LAZY>(p, s, "ng_rmsnorm_gemm_lazy");
}

ng_status ng_lazy_fold_affine(const ng_bf16* B, const ng_bf16* gamma, const ng_bf16* beta,
                        ng_bf16* B_folded, float* bias, int64_t K, int64_t N, int b_layout,
                        void* stream) {
  if (!B || !B_folded) return fail(NG_ERR_INVALID_ARG, "B and B_folded must be non-NULL");
  if (!aligned(B, 16) || !aligned(B_folded, 16))
    return fail(NG_ERR_INVALID_ARG, "B and B_folded must be 16-byte aligned");
  if (K < 1 || N < 1 || K > kMaxDim || N > kMaxDim)
    return fail(NG_ERR_INVALID_ARG, "need 1 <= K, N <= 2^24 (got K=%lld N=%lld)", (long long)K,
                (long long)N);
  if (b_layout != NG_B_KN && b_layout != NG_B_NK)
    return fail(NG_ERR_INVALID_ARG, "b_layout must be NG_B_KN or NG_B_NK (got %d)", b_layout);
  ng_status st = check_vec(gamma, "gamma", 16);
  if (!st) st = check_vec(beta, "beta", 16);
  if (!st) st = check_vec(bias, "bias", 4);
  if (st) return st;
  if (N % 8 != 0 || K % 8 != 0)
    return fail(NG_ERR_UNSUPPORTED, "N and K must be multiples of 8 (got N=%lld K=%lld)",
                (long long)N, (long long)K);
  if (K * N >= (int64_t(1) << 31) * 8)
    return fail(NG_ERR_UNSUPPORTED, "B has more than 2^34 elements");
  ng::FoldParams p{};
  p.B = B;
  p.gamma = gamma;
  p.beta = beta;
  p.B_folded = B_folded;
  p.bias = bias;
  p.K = K;
  p.N = N;
  p.nk = b_layout == NG_B_NK;
  hipStream_t s = (hipStream_t)stream;
  // the bias reads B before B_folded may overwrite it (same stream, in order)
  if (bias) {
    const unsigned grid = (unsigned)(p.nk ? (N + 3) / 4 : (N + 63) / 64);
    hipLaunchKernelGGL(ng::fold_bias_kernel, dim3(grid), dim3(256), 0, s, p);
    st = launched("ng_lazy_fold_affine (bias)");
    if (st) return st;
  }
  const int64_t chunks = K * N / 8;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(ng::fold_gamma_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return launched("ng_lazy_fold_affine");
}

ng_status ng_rmsnorm_gemm_lazy_affine(const ng_bf16* A, const ng_bf16* B_folded, const float* bias,
                                ng_bf16* C, int64_t M, int64_t N, int64_t K, int b_layout,
                                float eps, float* rstd_out, void* stream) {
  ng_status st = check_gemm(A, B_folded, C, M, N, K, b_layout);
  if (!st) st = check_eps(eps);
  if (!st) st = check_vec(bias, "bias", 16);
  if (!st) st = check_vec(rstd_out, "rstd_out", 4);
  if (st) return st;
  if (M == 0) return ok();
  ng::GemmParams p = make_params(A, B_folded, C, M, N, K, eps);
  p.rstd_out = rstd_out;
  p.bias = bias;
  hipStream_t s = (hipStream_t)stream;
  const bool kn = b_layout == NG_B_KN;
  const char* what = "ng_rmsnorm_gemm_lazy_affine";
  if (!bias) {
    if (N <= 128)
      return kn ? launch_grid<TRow128<true>, ng::EPI_LAZY>(p, s, what)
                : launch_grid<TRow128<false>, ng::EPI_LAZY>(p, s, what);
    return kn ? launch_persistent<TLarge<true>, ng::EPI_LAZY>(p, s, what)
              : launch_persistent<TLarge<false>, ng::EPI_LAZY>(p, s, what);
  }
  if (N <= 128)
    return kn ? launch_grid<TRow128<true>, ng::EPI_LAZY_BIAS>(p, s, what)
              : launch_grid<TRow128<false>, ng::EPI_LAZY_BIAS>(p, s, what);
  return kn ? launch_persistent<TLarge<true>, ng::EPI_LAZY_BIAS>(p, s, what)
            : launch_persistent<TLarge<false>, ng::EPI_LAZY_BIAS>(p, s, what);
}

ng_status ng_gemm_rmsnorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* gamma, ng_bf16* C,
                    int64_t M, int64_t N, int64_t K, int b_layout, float eps, float* rstd_out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_norm(A, B, nullptr, gamma, nullptr, C, nullptr, M, N, K, b_layout, eps, nullptr,
                   rstd_out, workspace, workspace_bytes, (hipStream_t)stream, ng::NORM_RMS, false,
                   "ng_gemm_rmsnorm");
}

ng_status ng_gemm_layernorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* gamma,
                      const ng_bf16* beta, ng_bf16* C, int64_t M, int64_t N, int64_t K,
                      int b_layout, float eps, float* mean_out, float* rstd_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return gemm_norm(A, B, nullptr, gamma, beta, C, nullptr, M, N, K, b_layout, eps, mean_out,
                   rstd_out, workspace, workspace_bytes, (hipStream_t)stream, ng::NORM_LAYER, false,
                   "ng_gemm_layernorm");
}

ng_status ng_gemm_add_rmsnorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* R,
                        const ng_bf16* gamma, ng_bf16* C, ng_bf16* S_out, int64_t M, int64_t N,
                        int64_t K, int b_layout, float eps, float* rstd_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return gemm_norm(A, B, R, gamma, nullptr, C, S_out, M, N, K, b_layout, eps, nullptr, rstd_out,
                   workspace, workspace_bytes, (hipStream_t)stream, ng::NORM_RMS, true,
                   "ng_gemm_add_rmsnorm");
}

ng_status ng_gemm_add_layernorm(const ng_bf16* A, const ng_bf16* B, const ng_bf16* R,
                          const ng_bf16* gamma, const ng_bf16* beta, ng_bf16* C, ng_bf16* S_out,
                          int64_t M, int64_t N, int64_t K, int b_layout, float eps,
                          float* mean_out, float* rstd_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return gemm_norm(A, B, R, gamma, beta, C, S_out, M, N, K, b_layout, eps, mean_out, rstd_out,
                   workspace, workspace_bytes, (hipStream_t)stream, ng::NORM_LAYER, true,
                   "ng_gemm_add_layernorm");
}

ng_status ng_gemm(const ng_bf16* A, const ng_bf16* B, ng_bf16* C, int64_t M, int64_t N, int64_t K,
            int b_layout, void* stream) {
  ng_status st = check_gemm(A, B, C, M, N, K, b_layout);
  if (st) return st;
  if (M == 0) return ok();
  ng::GemmParams p = make_params(A, B, C, M, N, K, 0.f);
  hipStream_t s = (hipStream_t)stream;
  const bool kn = b_layout == NG_B_KN;
  if (N <= 128)
    return kn ? launch_grid<TRow128<true>, ng::EPI_NONE>(p, s, "ng_gemm")
              : launch_grid<TRow128<false>, ng::EPI_NONE>(p, s, "ng_gemm");
  return kn ? launch_persistent<TLarge<true>, ng::EPI_NONE>(p, s, "ng_gemm")
            : launch_persistent<TLarge<false>, ng::EPI_NONE>(p, s, "ng_gemm");
}

}  // extern "C"

namespace {

// Launch shape of the norm kernel for p.cols (rows of up to 65536 columns).
ng_status launch_norm_rows(const ng::NormParams& p, hipStream_t s, bool residual, const char* what) {
  const int64_t rows = p.rows;
  const int64_t nch = p.cols / 8;
#define NG_NORM_LAUNCH(LPR, CPL)                                                              \
  do {                                                                                        \
    const unsigned grid = (unsigned)((rows + (256 / LPR) - 1) / (256 / LPR));                 \
    if (residual)                                                                             \
      hipLaunchKernelGGL((ng::norm_kernel<LPR, CPL, true>), dim3(grid), dim3(256), 0, s, p);  \
    else                                                                                      \
      hipLaunchKernelGGL((ng::norm_kernel<LPR, CPL, false>), dim3(grid), dim3(256), 0, s, p); \
    return launched(what);                                                                    \
  } while (0)
  if (nch <= 16) NG_NORM_LAUNCH(16, 1);
  if (nch <= 32) NG_NORM_LAUNCH(32, 1);
  if (nch <= 64) NG_NORM_LAUNCH(64, 1);
  if (nch <= 128) NG_NORM_LAUNCH(64, 2);
  if (nch <= 256) NG_NORM_LAUNCH(64, 4);
  if (nch <= 512) NG_NORM_LAUNCH(128, 4);
  if (nch <= 1024) NG_NORM_LAUNCH(256, 4);
  if (nch <= 2048) NG_NORM_LAUNCH(256, 8);
  if (nch <= 4096) NG_NORM_LAUNCH(256, 16);
  NG_NORM_LAUNCH(256, 32);
#undef NG_NORM_LAUNCH
}

// Shared by ng_norm and ng_add_norm (R non-NULL).
ng_status norm_rows(const ng_bf16* X, const ng_bf16* R, const ng_bf16* gamma, const ng_bf16* beta,
              ng_bf16* Y, ng_bf16* S_out, int64_t rows, int64_t cols, int kind, float eps,
              float* mean_out, float* rstd_out, hipStream_t s, bool residual, const char* what) {
  if (rows != 0 && (!X || !Y)) return fail(NG_ERR_INVALID_ARG, "X and Y must be non-NULL");
  if (!aligned(X, 16) || !aligned(Y, 16))
    return fail(NG_ERR_INVALID_ARG, "X and Y must be 16-byte aligned");
  if (residual) {
    if (rows != 0 && !R) return fail(NG_ERR_INVALID_ARG, "R must be non-NULL");
    if (!aligned(R, 16) || !aligned(S_out, 16))
      return fail(NG_ERR_INVALID_ARG, "R and S_out must be 16-byte aligned");
    if (S_out && rows != 0 && S_out == Y)
      return fail(NG_ERR_INVALID_ARG, "S_out and Y must be different buffers");
  }
  if (rows < 0 || cols < 1 || rows > kMaxDim * 64)
    return fail(NG_ERR_INVALID_ARG, "need rows >= 0 and cols >= 1");
  if (kind != NG_NORM_RMS && kind != NG_NORM_LAYER)
    return fail(NG_ERR_INVALID_ARG, "kind must be NG_NORM_RMS or NG_NORM_LAYER");
  if (kind == NG_NORM_RMS && mean_out)
    return fail(NG_ERR_INVALID_ARG, "RMSNorm has no mean output");
  ng_status st = check_eps(eps);
  if (!st) st = check_vec(gamma, "gamma", 16);
  if (!st) st = check_vec(beta, "beta", 16);
  if (!st) st = check_vec(mean_out, "mean_out", 4);
  if (!st) st = check_vec(rstd_out, "rstd_out", 4);
  if (st) return st;
  if (cols % 8 != 0 || cols > 65536)
    return fail(NG_ERR_UNSUPPORTED, "cols must be a multiple of 8 and at most 65536");
  if (rows == 0) return ok();
  ng::NormParams p{};
  p.X = X;
  p.R = R;
  p.S_out = S_out;
  p.gamma = gamma;
  p.beta = beta;
  p.Y = Y;
  p.mean_out = mean_out;
  p.rstd_out = rstd_out;
  p.rows = (int)rows;
  p.cols = (int)cols;
  p.kind = kind;
  p.eps = eps;
  return launch_norm_rows(p, s, residual, what);
}

}  // namespace

extern "C" {

ng_status ng_norm(const ng_bf16* X, const ng_bf16* gamma, const ng_bf16* beta, ng_bf16* Y,
            int64_t rows, int64_t cols, int kind, float eps, float* mean_out, float* rstd_out,
            void* stream) {
  return norm_rows(X, nullptr, gamma, beta, Y, nullptr, rows, cols, kind, eps, mean_out,
                   rstd_out, (hipStream_t)stream, false, "ng_norm");
}

ng_status ng_add_norm(const ng_bf16* X, const ng_bf16* R, const ng_bf16* gamma, const ng_bf16* beta,
                ng_bf16* Y, ng_bf16* S_out, int64_t rows, int64_t cols, int kind, float eps,
                float* mean_out, float* rstd_out, void* stream) {
  return norm_rows(X, R, gamma, beta, Y, S_out, rows, cols, kind, eps, mean_out, rstd_out,
                   (hipStream_t)stream, true, "ng_add_norm");
}

ng_status ng_layernorm_gemm_fold(const ng_bf16* B, const ng_bf16* gamma, const ng_bf16* beta,
                           ng_bf16* B_folded, float* colsum, float* bias, int64_t K, int64_t N,
                           int b_layout, void* stream) {
  if (!colsum) return fail(NG_ERR_INVALID_ARG, "colsum must be non-NULL");
  if (!aligned(colsum, 16)) return fail(NG_ERR_INVALID_ARG, "colsum must be 16-byte aligned");
  if (bias && !aligned(bias, 16)) return fail(NG_ERR_INVALID_ARG, "bias must be 16-byte aligned");
  if (beta && !bias) return fail(NG_ERR_INVALID_ARG, "beta needs a bias output");
  // bias = beta^T B (before B_folded may overwrite B), then B' = diag(gamma) B
  ng_status st = ng_lazy_fold_affine(B, gamma, beta, B_folded, bias, K, N, b_layout, stream);
  if (st) return st;
  // colsum = 1^T B' over the folded (bf16-rounded) weights the product uses
  ng::FoldParams p{};
  p.B = B_folded;
  p.bias = colsum;
  p.K = K;
  p.N = N;
  p.nk = b_layout == NG_B_NK;
  p.ones = 1;
  const unsigned grid = (unsigned)(p.nk ? (N + 3) / 4 : (N + 63) / 64);
  hipLaunchKernelGGL(ng::fold_bias_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, p);
  return launched("ng_layernorm_gemm_fold");
}

ng_status ng_layernorm_gemm_prenorm(const ng_bf16* A, const ng_bf16* B_folded, const float* colsum,
                              const float* bias, ng_bf16* C, int64_t M, int64_t N, int64_t K,
                              int b_layout, float eps, float* mean, float* rstd, void* stream) {
  ng_status st = check_gemm(A, B_folded, C, M, N, K, b_layout);
  if (!st) st = check_eps(eps);
  if (st) return st;
  if (!colsum || !aligned(colsum, 16))
    return fail(NG_ERR_INVALID_ARG, "colsum must be non-NULL and 16-byte aligned");
  if (bias && !aligned(bias, 16)) return fail(NG_ERR_INVALID_ARG, "bias must be 16-byte aligned");
  if (M != 0 && (!mean || !rstd)) return fail(NG_ERR_INVALID_ARG, "mean and rstd must be non-NULL");
  if (!aligned(mean, 4) || !aligned(rstd, 4))
    return fail(NG_ERR_INVALID_ARG, "mean and rstd must be 4-byte aligned");
  if (K > 65536) return fail(NG_ERR_UNSUPPORTED, "K must be at most 65536 (row statistics)");
  if (M == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  // stage 1: mean and rstd of every row of A (no normalized output)
  ng::NormParams q{};
  q.X = A;
  q.mean_out = mean;
  q.rstd_out = rstd;
  q.rows = (int)M;
  q.cols = (int)K;
  q.kind = ng::NORM_LAYER;
  q.eps = eps;
  const char* what = "ng_layernorm_gemm_prenorm";
  st = launch_norm_rows(q, s, false, what);
  if (st) return st;
  // stage 2: the product with the norm applied through it
  ng::GemmParams p = make_params(A, B_folded, C, M, N, K, eps);
  p.colsum = colsum;
  p.bias = bias;
  p.row_mean = mean;
  p.row_rstd = rstd;
  const bool kn = b_layout == NG_B_KN;
  if (N <= 128)
    return kn ? launch_grid<TRow128<true>, ng::EPI_PRE_LN>(p, s, what)
              : launch_grid<TRow128<false>, ng::EPI_PRE_LN>(p, s, what);
  return kn ? launch_persistent<TLarge<true>, ng::EPI_PRE_LN>(p, s, what)
            : launch_persistent<TLarge<false>, ng::EPI_PRE_LN>(p, s, what);
}

// The input gradient; with scaled_out, the kernel also writes rstd * dC
// (the regrouped weight gradient's operand).
static ng_status lazy_backward_input(const ng_bf16* dC, const ng_bf16* B, const ng_bf16* A,
                                     const float* rstd, ng_bf16* dA, ng_bf16* scaled_out,
                                     int64_t M, int64_t N, int64_t K, int b_layout,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     const char* what) {
  // dA_hat = dC [M, N] @ B^T [N, K]: the product's output width is the
  // forward K and its reduction the forward N; B^T is B read in the other
  // layout
  if (b_layout != NG_B_KN && b_layout != NG_B_NK)
    return fail(NG_ERR_INVALID_ARG, "b_layout must be NG_B_KN or NG_B_NK (got %d)", b_layout);
  const int lay = b_layout == NG_B_KN ? NG_B_NK : NG_B_KN;
  ng_status st = check_gemm(dC, B, dA, M, K, N, lay);
  if (st) return st;
  if (M != 0 && (!A || !rstd)) return fail(NG_ERR_INVALID_ARG, "A and rstd must be non-NULL");
  if (!aligned(A, 16)) return fail(NG_ERR_INVALID_ARG, "A must be 16-byte aligned");
  if (!aligned(rstd, 4)) return fail(NG_ERR_INVALID_ARG, "rstd must be 4-byte aligned");
  const bool local = K <= row_local_max();
  if (!local && M > 0) {
    const size_t need = xwg_bytes(M, K);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
      return fail(NG_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed, got %zu",
                  need, workspace_bytes);
  }
  if (M == 0) return ok();
  ng::GemmParams p = make_params(dC, B, dA, M, K, N, 0.f);
  p.Xin = A;
  p.row_rstd = rstd;
  p.scaled_out = (uint16_t*)scaled_out;
  p.ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const bool kn = lay == NG_B_KN;
  if (local && K <= 128)
    return kn ? launch_grid<TRow128<true>, ng::EPI_LAZY_BWD>(p, s, what)
              : launch_grid<TRow128<false>, ng::EPI_LAZY_BWD>(p, s, what);
  if (local)
    return kn ? launch_grid<TRow256<true>, ng::EPI_LAZY_BWD>(p, s, what)
              : launch_grid<TRow256<false>, ng::EPI_LAZY_BWD>(p, s, what);
  return kn ? launch_xwg<TLarge<true>, false, false, true>(p, s, what)
            : launch_xwg<TLarge<false>, false, false, true>(p, s, what);
}

ng_status ng_rmsnorm_gemm_lazy_backward_input(const ng_bf16* dC, const ng_bf16* B, const ng_bf16* A,
                                         const float* rstd, ng_bf16* dA, int64_t M, int64_t N,
                                         int64_t K, int b_layout, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return lazy_backward_input(dC, B, A, rstd, dA, nullptr, M, N, K, b_layout, workspace,
                             workspace_bytes, stream, "ng_rmsnorm_gemm_lazy_backward_input");
}

ng_status ng_rmsnorm_gemm_lazy_backward(const ng_bf16* dC, const ng_bf16* B, const ng_bf16* A,
                                   const float* rstd, ng_bf16* dA, ng_bf16* dB,
                                   ng_bf16* dC_scaled, int64_t M, int64_t N, int64_t K,
                                   int b_layout, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const char* what = "ng_rmsnorm_gemm_lazy_backward";
  if (!dB || (M != 0 && !dC_scaled))
    return fail(NG_ERR_INVALID_ARG, "dB and dC_scaled must be non-NULL");
  if (!aligned(dB, 16) || !aligned(dC_scaled, 16))
    return fail(NG_ERR_INVALID_ARG, "dB and dC_scaled must be 16-byte aligned");
  if (M > 0 && N > 0 && K > 0 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim) {
    // the scratch is distinct from every other argument
    const uintptr_t sc = (uintptr_t)dC_scaled, sce = sc + (uintptr_t)(M * N * 2);
    const struct { const void* p; int64_t bytes; } others[] = {
        {dC, M * N * 2}, {B, K * N * 2}, {A, M * K * 2}, {rstd, M * 4}, {dA, M * K * 2},
        {dB, K * N * 2}, {workspace, (int64_t)workspace_bytes}};
    for (const auto& o : others) {
      const uintptr_t b = (uintptr_t)o.p, e = b + (uintptr_t)o.bytes;
      if (o.p && b < sce && sc < e)
        return fail(NG_ERR_INVALID_ARG, "dC_scaled must not overlap the other arguments");
    }
  }
  // dA, and rstd * dC into dC_scaled (the checks of the input gradient apply)
  ng_status st = lazy_backward_input(dC, B, A, rstd, dA, dC_scaled, M, N, K, b_layout, workspace,
                                     workspace_bytes, stream, what);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  if (M == 0) {
    // an empty sum over rows: dB = 0
    const size_t n16 = (size_t)(K * N) / 8;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(ng::fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (ng::u32x4*)dB, n16, (uint32_t*)nullptr, (size_t)0);
    return launched(what);
  }
  // dB = A^T (rstd * dC) over the forward rows: [K, N] = gemm_at(A, dC_scaled)
  // for B stored [K, N]; [N, K] = gemm_at(dC_scaled, A) for B stored [N, K]
  ng::GemmParams p{};
  p.C = (uint16_t*)dB;
  p.K = (int)M;
  p.spin_limit = wait_spins();
  if (b_layout == NG_B_KN) {
    p.A = (const uint16_t*)A;
    p.B = (const uint16_t*)dC_scaled;
    p.M = (int)K;
    p.N = (int)N;
  } else {
    p.A = (const uint16_t*)dC_scaled;
    p.B = (const uint16_t*)A;
    p.M = (int)N;
    p.N = (int)K;
  }
  return launch_persistent<TWgrad<0>, ng::EPI_NONE>(p, s, what);
}

ng_status ng_rmsnorm_gemm_lazy_backward_weight(const ng_bf16* A, const ng_bf16* dC, const float* rstd,
                                          ng_bf16* dB, int64_t M, int64_t N, int64_t K,
                                          int b_layout, void* stream) {
  if (M != 0 && (!A || !dC || !rstd)) return fail(NG_ERR_INVALID_ARG, "A, dC and rstd must be non-NULL");
  if (!dB) return fail(NG_ERR_INVALID_ARG, "dB must be non-NULL");
  if (!aligned(A, 16) || !aligned(dC, 16) || !aligned(dB, 16))
    return fail(NG_ERR_INVALID_ARG, "A, dC and dB must be 16-byte aligned");
  if (!aligned(rstd, 4)) return fail(NG_ERR_INVALID_ARG, "rstd must be 4-byte aligned");
  if (M < 0 || N < 1 || K < 1)
    return fail(NG_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1 (got M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(NG_ERR_INVALID_ARG, "M, N, K must be at most 2^24");
  if (b_layout != NG_B_KN && b_layout != NG_B_NK)
    return fail(NG_ERR_INVALID_ARG, "b_layout must be NG_B_KN or NG_B_NK (got %d)", b_layout);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(NG_ERR_UNSUPPORTED, "N and K must be multiples of 8 (got N=%lld K=%lld)",
                (long long)N, (long long)K);
  if (M * K >= (int64_t(1) << 31) * 8 || M * N >= (int64_t(1) << 31) * 8 ||
      K * N >= (int64_t(1) << 31) * 8)
    return fail(NG_ERR_UNSUPPORTED, "a matrix has more than 2^34 elements");
  hipStream_t s = (hipStream_t)stream;
  const char* what = "ng_rmsnorm_gemm_lazy_backward_weight";
  if (M == 0) {
    // an empty sum over rows: dB = 0
    const size_t n16 = (size_t)(K * N) / 8;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(ng::fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (ng::u32x4*)dB, n16, (uint32_t*)nullptr, (size_t)0);
    return launched(what);
  }
  // B [K, N]: dB = A_hat^T @ dC, the product over the forward rows with A read
  // transposed and scaled.  B [N, K]: dB = dC^T @ A_hat, dC read transposed
  // and A scaled on the other side.
  ng::GemmParams p{};
  p.row_rstd = rstd;
  p.C = (uint16_t*)dB;
  p.K = (int)M;
  p.spin_limit = wait_spins();
  if (b_layout == NG_B_KN) {
    p.A = (const uint16_t*)A;
    p.B = (const uint16_t*)dC;
    p.M = (int)K;
    p.N = (int)N;
    return launch_persistent<TWgrad<1>, ng::EPI_NONE>(p, s, what);
  }
  p.A = (const uint16_t*)dC;
  p.B = (const uint16_t*)A;
  p.M = (int)N;
  p.N = (int)K;
  return launch_persistent<TWgrad<2>, ng::EPI_NONE>(p, s, what);
}

ng_status ng_gemm_at(const ng_bf16* A, const ng_bf16* B, ng_bf16* C, int64_t M, int64_t N, int64_t K,
               void* stream) {
  if (M != 0 && N != 0 && (!A || !B || !C))
    return fail(NG_ERR_INVALID_ARG, "A, B and C must be non-NULL");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16))
    return fail(NG_ERR_INVALID_ARG, "A, B and C must be 16-byte aligned");
  if (M < 1 || N < 1 || K < 1)
    return fail(NG_ERR_INVALID_ARG, "need M, N, K >= 1 (got M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(NG_ERR_INVALID_ARG, "M, N, K must be at most 2^24");
  if (M % 8 != 0 || N % 8 != 0)
    return fail(NG_ERR_UNSUPPORTED, "M and N must be multiples of 8 (got M=%lld N=%lld)",
                (long long)M, (long long)N);
  if (M * K >= (int64_t(1) << 31) * 8 || N * K >= (int64_t(1) << 31) * 8 ||
      M * N >= (int64_t(1) << 31) * 8)
    return fail(NG_ERR_UNSUPPORTED, "a matrix has more than 2^34 elements");
  ng::GemmParams p{};
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.C = (uint16_t*)C;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.spin_limit = wait_spins();
  return launch_persistent<TWgrad<0>, ng::EPI_NONE>(p, (hipStream_t)stream, "ng_gemm_at");
}

ng_status ng_rmsnorm_backward(const ng_bf16* dY, const ng_bf16* X, const float* rstd, ng_bf16* dX,
                        int64_t rows, int64_t cols, void* stream) {
  if (rows != 0 && (!dY || !X || !rstd || !dX))
    return fail(NG_ERR_INVALID_ARG, "dY, X, rstd and dX must be non-NULL");
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(dX, 16))
    return fail(NG_ERR_INVALID_ARG, "dY, X and dX must be 16-byte aligned");
  if (!aligned(rstd, 4)) return fail(NG_ERR_INVALID_ARG, "rstd must be 4-byte aligned");
  if (rows < 0 || cols < 1 || rows > kMaxDim * 64)
    return fail(NG_ERR_INVALID_ARG, "need rows >= 0 and cols >= 1");
  if (cols % 8 != 0 || cols > 65536)
    return fail(NG_ERR_UNSUPPORTED, "cols must be a multiple of 8 and at most 65536");
  if (rows == 0) return ok();
  ng::NormBwdParams p{};
  p.dY = dY;
  p.X = X;
  p.rstd = rstd;
  p.dX = dX;
  p.rows = (int)rows;
  p.cols = (int)cols;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = cols / 8;
#define NG_NORM_BWD_LAUNCH(LPR, CPL)                                                      \
  do {                                                                                    \
    const unsigned grid = (unsigned)((rows + (256 / LPR) - 1) / (256 / LPR));             \
    hipLaunchKernelGGL((ng::norm_bwd_kernel<LPR, CPL>), dim3(grid), dim3(256), 0, s, p);  \
    return launched("ng_rmsnorm_backward");                                               \
  } while (0)
  if (nch <= 16) NG_NORM_BWD_LAUNCH(16, 1);
  if (nch <= 32) NG_NORM_BWD_LAUNCH(32, 1);
  if (nch <= 64) NG_NORM_BWD_LAUNCH(64, 1);
  if (nch <= 128) NG_NORM_BWD_LAUNCH(64, 2);
  if (nch <= 256) NG_NORM_BWD_LAUNCH(64, 4);
  if (nch <= 512) NG_NORM_BWD_LAUNCH(128, 4);
  if (nch <= 1024) NG_NORM_BWD_LAUNCH(256, 4);
  if (nch <= 2048) NG_NORM_BWD_LAUNCH(256, 8);
  if (nch <= 4096) NG_NORM_BWD_LAUNCH(256, 16);
  NG_NORM_BWD_LAUNCH(256, 32);
#undef NG_NORM_BWD_LAUNCH
}

size_t ng_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
  // the Lazy backward normalizes rows of length K (the forward A's rows)
  if (op == NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT) N = K;
  if (op != NG_OP_GEMM_RMSNORM && op != NG_OP_GEMM_LAYERNORM && op != NG_OP_GEMM_ADD_RMSNORM &&
      op != NG_OP_GEMM_ADD_LAYERNORM && op != NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT)
    return 0;
  if (M <= 0 || N <= row_local_max() || M > kMaxDim || N > kMaxDim) return 0;
  return xwg_bytes(M, N);
}

ng_status ng_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256))
    return fail(NG_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes % 4 != 0) return fail(NG_ERR_INVALID_ARG, "workspace size must be a multiple of 4");
  if (workspace_bytes == 0) return ok();
  const size_t n16 = workspace_bytes / 16;
  const size_t ntail = (workspace_bytes % 16) / 4;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ng::fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, (ng::u32x4*)workspace, n16,
                     (uint32_t*)((char*)workspace + n16 * 16), ntail);
  return launched("ng_workspace_reset");
}

ng_status ng_workspace_status(const void* workspace, void* stream) {
  if (!workspace || !aligned(workspace, 256))
    return fail(NG_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(NG_ERR_HIP, "stream sync failed: %s", hipGetErrorString(e));
  int word = 0;
  e = hipMemcpy(&word, workspace, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(NG_ERR_HIP, "reading the error word failed: %s", hipGetErrorString(e));
  if (word != 0) return fail(NG_ERR_TIMEOUT, "a cross-workgroup wait timed out");
  return ok();
}

const char* ng_status_string(ng_status status) {
  switch (status) {
    case NG_OK: return "NG_OK";
    case NG_ERR_INVALID_ARG: return "NG_ERR_INVALID_ARG";
    case NG_ERR_UNSUPPORTED: return "NG_ERR_UNSUPPORTED";
    case NG_ERR_WORKSPACE: return "NG_ERR_WORKSPACE";
    case NG_ERR_HIP: return "NG_ERR_HIP";
    case NG_ERR_TIMEOUT: return "NG_ERR_TIMEOUT";
    default: return "NG_ERR_UNKNOWN";
  }
}

const char* ng_last_error(void) { return g_err; }

ng_status ng_set_debug_option(int option, int64_t value) {
  switch (option) {
    case NG_DEBUG_WAIT_SPINS:
      if (value < -1 || value > (int64_t(1) << 30))
        return fail(NG_ERR_INVALID_ARG, "wait bound must be -1 or in 0 .. 2^30");
      g_wait_spins.store((int)value, std::memory_order_relaxed);
      return ok();
    case NG_DEBUG_ROW_LOCAL_MAX:
      if (value < -1 || value > 256)
        return fail(NG_ERR_INVALID_ARG, "row-local maximum must be -1 or in 0 .. 256");
      g_row_local_max.store((int)value, std::memory_order_relaxed);
      return ok();
    case NG_DEBUG_TILE_ORDER:
      if (value != NG_TILE_ORDER_NATURAL && value != NG_TILE_ORDER_REVERSED &&
          value != NG_TILE_ORDER_SHUFFLED)
        return fail(NG_ERR_INVALID_ARG, "unknown tile order %lld", (long long)value);
      g_tile_order.store((int)value, std::memory_order_relaxed);
      return ok();
    case NG_DEBUG_K_WALK:
      if (value != NG_K_WALK_AUTO && value != NG_K_WALK_UPWARD && value != NG_K_WALK_ALTERNATE)
        return fail(NG_ERR_INVALID_ARG, "unknown k-walk mode %lld", (long long)value);
      g_k_walk.store((int)value, std::memory_order_relaxed);
      return ok();
    default:
      return fail(NG_ERR_INVALID_ARG, "unknown debug option %d", option);
  }
}

}  // extern "C"
