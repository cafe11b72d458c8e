// libtpshard: C ABI of one tensor-parallel rank's Megatron-style layer shard
// on gfx950.  Argument validation, tile-configuration choice and kernel
// launches on the caller's stream; the kernels live in the headers next to
// this file.  The interface is declared and documented in include/tp_shard.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "../../include/tp_shard.h"
#include "attention.hpp"
#include "attention_bwd.hpp"
#include "elementwise.hpp"
#include "epilogues.hpp"
#include "gemm_dma.hpp"
#include "gemm_common.hpp"
#include "gemm_simt.hpp"

using namespace tp;

namespace {

constexpr int kNumCUs = 256;

// Profiling aid (tp_profile_arm): events recorded around the next kernels.
// `armed` lets an unarmed launch skip the lock; the table itself is guarded
// by `mu`, so concurrent launches each claim a distinct slot.
struct ProfileHook {
  std::mutex mu;
  std::atomic<bool> armed{false};
  hipEvent_t ev[64];
  int n_kernels = 0;  // kernels to bracket
  int next = 0;       // next slot to hand out
} g_prof;

// Opens a profiling scope over the kernels launched while it lives, with the
// next armed event pair, if any: tp_launch attaches the events to those
// kernels' dispatches.  A scope that launches nothing records both events on
// the stream.
struct Probe {
  hipStream_t st;
  tp::LaunchEvents ev;
  tp::LaunchEvents* outer = nullptr;
  bool open = false;
  explicit Probe(hipStream_t s) : st(s) {
    if (!g_prof.armed.load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.next < g_prof.n_kernels) {
      const int idx = g_prof.next++;
      ev.start = g_prof.ev[2 * idx];
      ev.stop = g_prof.ev[2 * idx + 1];
      outer = tp::g_launch_events;
      tp::g_launch_events = &ev;
      open = true;
      if (g_prof.next == g_prof.n_kernels) g_prof.armed.store(false, std::memory_order_release);
    }
  }
  ~Probe() {
    if (!open) return;
    tp::g_launch_events = outer;
    if (!ev.started) {
      hipEventRecord(ev.start, st);
      hipEventRecord(ev.stop, st);
    }
  }
};

// Process-wide launch options (tp_set_options): the tile choice and the
// splits of last rounds and heavy attention blocks.
std::atomic<int> g_tile{TP_TILE_AUTO};
std::atomic<int> g_split{1};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool fits_int(int64_t v) { return v >= 0 && v <= INT32_MAX; }

int check_dropout(float p, uint32_t* thr, float* scale) {
  if (!(p >= 0.0f && p < 1.0f)) return TP_EINVAL;
  // floor(p * 2^32), p taken exactly as the float it is.
  *thr = (uint32_t)std::floor((double)p * 4294967296.0);
  *scale = 1.0f / (1.0f - p);
  return TP_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_EHIP; }

GemmProblem problem(int M, int N, int K, const void* A, int64_t lda, const void* B0, const void* B1, int64_t ldb) {
  GemmProblem p{};
  p.M = M;
  p.N = N;
  p.nseg = 1;
  p.K[0] = K;
  p.K[1] = 0;
  p.A[0] = static_cast<const uint16_t*>(A);
  p.B[0][0] = static_cast<const uint16_t*>(B0);
  p.B[0][1] = static_cast<const uint16_t*>(B1);
  p.lda[0] = p.lda[1] = lda;
  p.ldb[0] = p.ldb[1] = ldb;
  return p;
}

// Tile choice: the large tile (one work-group per CU) unless it would leave
// more than ~44% of the 256 CUs without a tile; then the quarter-size tile,
// of which two work-groups share a CU.  Measured on gfx950: with 160 or more
// large tiles the large tile wins even though some CUs idle (a partly idle
// chip clocks higher), with 128 or fewer the small tile wins.
// tp_set_options can force one tile shape (the tests cover every shape at
// small sizes) and turn off the split of a GEMM's last round (in K for a
// single GEMM, in N for a pair) and the splits of the attention kernels'
// heaviest key and query blocks (the tests compare both ways).
bool split_tail_enabled() { return g_split.load(std::memory_order_relaxed) != 0; }

int64_t tile_count(const GemmProblem& p, int bm, int bn) {
  return (int64_t)((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
}
bool use_small_tile(int64_t big) {
  switch (g_tile.load(std::memory_order_relaxed)) {
    case TP_TILE_LARGE: return false;
    case TP_TILE_SMALL:
    case TP_TILE_TINY: return true;
    default: return big < (int64_t)kNumCUs * 9 / 16;
  }
}
// Among launches that take the small tile, those whose small tiles would
// fill fewer than half of the 512 work-group slots (two per CU) take the
// 64 x 64 tile of four 32 x 32 waves instead (single-B epilogues only): small
// GEMMs with few tiles are bound by the latency of their K loop, and four
// times the work-groups hide it.  TP_TILE_TINY forces it.
bool use_tiny_tile(int64_t small) {
  switch (g_tile.load(std::memory_order_relaxed)) {
    case TP_TILE_TINY: return true;
    case TP_TILE_LARGE:
    case TP_TILE_SMALL: return false;
    default: return small < (int64_t)kNumCUs;
  }
}

template <int AL, int BL, class Epi>
hipError_t gemm_bf16(const GemmProblem& p, const Epi& epi, hipStream_t st) {
  constexpr int BN = Epi::NB == 1 ? 256 : 128;
  Probe pr(st);
  if (use_small_tile(tile_count(p, 256, BN))) {
    if constexpr (Epi::NB == 1) {
      if (use_tiny_tile(tile_count(p, 128, 128))) return launch_gemm_dma<64, 64, 2, 2, 64, AL, BL>(p, epi, st);
    }
    return launch_gemm_dma<128, BN / 2, 2, 2, 64, AL, BL>(p, epi, st);
  }
  return launch_gemm_dma<256, BN, 4, 2, 64, AL, BL>(p, epi, st);
}

// gemm_bf16 with device memory `scratch` (scratch_bytes bytes, 16-byte
// aligned) that the call may overwrite: when it is large enough and the large
// tile's last round would be at most half full, that round is split over K
// (SplitTail in gemm_dma.hpp).
template <int AL, int BL, class Epi>
hipError_t gemm_bf16_split(const GemmProblem& p, const Epi& epi, hipStream_t st, void* scratch, int64_t scratch_bytes) {
  constexpr int BN = Epi::NB == 1 ? 256 : 128;
  const int64_t need = split_tail_floats<256, BN, 64, Epi::NB>(p) * 4;
  if (!scratch || need == 0 || need > scratch_bytes || !split_tail_enabled() || use_small_tile(tile_count(p, 256, BN)))
    return gemm_bf16<AL, BL>(p, epi, st);
  Probe pr(st);
  return launch_gemm_dma_split<256, BN, 4, 2, 64, AL, BL>(p, epi, static_cast<float*>(scratch), st);
}

// Two independent bf16 GEMMs in one launch, p1's tiles dispatched first (the
// longer K first, so the shorter tiles fill the last round).  Both take the
// large tile unless their combined count of large tiles is below the
// crossover above, then both the small one.  A GEMM whose last round of tiles
// leaves CUs idle costs about a full round on its own (a power-limited chip
// clocks only a little higher when partly idle); in a pair the other
// problem's tiles take those CUs.  If the pair's last round is still at most
// half full, problem 2's last tile rows run as tiles of half the width,
// twice as many and half as long.
template <int AL1, int BL1, int AL2, int BL2, class E1, class E2>
hipError_t gemm_bf16_pair(const GemmProblem& p1, const E1& e1, const GemmProblem& p2, const E2& e2,
                          hipStream_t st) {
  constexpr int BN1 = E1::NB == 1 ? 256 : 128, BN2 = E2::NB == 1 ? 256 : 128;
  Probe pr(st);
  if (use_small_tile(tile_count(p1, 256, BN1) + tile_count(p2, 256, BN2))) {
    if constexpr (E1::NB == 1 && E2::NB == 1) {
      if (use_tiny_tile(tile_count(p1, 128, 128) + tile_count(p2, 128, 128)))
        return launch_gemm_dma_pair<gemm3::TileCfg<64, 64, 2, 2, 64, AL1, BL1>,
                                    gemm3::TileCfg<64, 64, 2, 2, 64, AL2, BL2>>(p1, e1, p2, e2, st);
    }
    return launch_gemm_dma_pair<gemm3::TileCfg<128, BN1 / 2, 2, 2, 64, AL1, BL1>,
                                gemm3::TileCfg<128, BN2 / 2, 2, 2, 64, AL2, BL2>>(p1, e1, p2, e2, st);
  }
  using C1 = gemm3::TileCfg<256, BN1, 4, 2, 64, AL1, BL1>;
  using C2 = gemm3::TileCfg<256, BN2, 4, 2, 64, AL2, BL2>;
  if constexpr (E2::NB == 1) {
    // last round at most half full: problem 2's last tile rows as 256 x 128 tiles
    const int rows2 = split_tail_enabled() ? pair_tail_rows<C1, C2>(p1, p2) : -1;
    if (rows2 >= 0) return launch_gemm_dma_pair_tail<C1, C2>(p1, e1, p2, e2, rows2, st);
  }
  return launch_gemm_dma_pair<C1, C2>(p1, e1, p2, e2, st);
}

// Operands stored in bf16 run on the matrix cores, operands stored in fp32 on
// the vector ALUs (S is the operand storage type).
template <class S, int AL, int BL, class Epi>
hipError_t gemm_any(const GemmProblem& p, const Epi& epi, hipStream_t st) {
  if constexpr (std::is_same_v<S, float>) {
    Probe pr(st);
    return launch_gemm_f32<AL, BL>(p, epi, st);
  }
  else
    return gemm_bf16<AL, BL>(p, epi, st);
}

unsigned grid_for(int64_t n_vec) {
  int64_t blocks = (n_vec + 255) / 256;
  if (blocks > 64 * kNumCUs) blocks = 64 * kNumCUs;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

template <class T>
hipError_t dropout_bwd(int64_t n, const void* dOut, uint32_t thr, float scale, uint64_t seed, void* dY, hipStream_t st) {
  const int64_t nv = n / Vec<T>::N;
  if (nv == 0) return hipSuccess;
  Probe pr(st);
  tp_launch(dropout_bwd_kernel<T>, dim3(grid_for(nv)), dim3(256), 0, st, nv, static_cast<const T*>(dOut), thr,
            scale, seed, static_cast<T*>(dY));
  return hipGetLastError();
}

template <class T>
hipError_t colsum(int64_t rows, int64_t cols, const void* X, float* out, hipStream_t st) {
  // column vectors per work-group: the most (up to 8) that still gives every CU one
  const int64_t nvec = cols / Vec<T>::N;
  if (nvec == 0) return hipSuccess;
  int cv = 8;
  while (cv > 1 && (nvec + cv - 1) / cv < kNumCUs) cv /= 2;
  const unsigned blocks = (unsigned)((nvec + cv - 1) / cv);
  Probe pr(st);
  const T* x = static_cast<const T*>(X);
  switch (cv) {
    case 8: tp_launch((colsum_kernel<T, 8>), dim3(blocks), dim3(256), 0, st, rows, cols, cols, x, out); break;
    case 4: tp_launch((colsum_kernel<T, 4>), dim3(blocks), dim3(256), 0, st, rows, cols, cols, x, out); break;
    case 2: tp_launch((colsum_kernel<T, 2>), dim3(blocks), dim3(256), 0, st, rows, cols, cols, x, out); break;
    default: tp_launch((colsum_kernel<T, 1>), dim3(blocks), dim3(256), 0, st, rows, cols, cols, x, out);
  }
  return hipGetLastError();
}

template <class T>
int mlp_fwd_impl(const tp_mlp_desc& d, int f, const void* X, const void* W1, const void* Wu, const void* b1,
                 const void* W2, void* saved, void* H, void* Z, hipStream_t st) {
  const int T_ = (int)d.tokens, h = (int)d.h;
  hipError_t e;
  if (d.act == TP_GELU) {
    EpiGeluFwd<T> epi{static_cast<T*>(saved), static_cast<T*>(H), static_cast<const T*>(b1), f, T_, f};
    e = gemm_any<T, KMAJOR, MNMAJOR>(problem(T_, f, h, X, h, W1, nullptr, f), epi, st);
  } else {
    T* G = static_cast<T*>(saved);
    EpiSwigluFwd<T> epi{G, G + (int64_t)T_ * f, static_cast<T*>(H), f, T_, f};
    if constexpr (std::is_same_v<T, float>)
      e = gemm_any<T, KMAJOR, MNMAJOR>(problem(T_, f, h, X, h, W1, Wu, f), epi, st);
    else  // Z_i is written only by the row GEMM below: until then it serves as scratch
      e = gemm_bf16_split<KMAJOR, MNMAJOR>(problem(T_, f, h, X, h, W1, Wu, f), epi, st, Z, (int64_t)T_ * h * 2);
  }
  if (e != hipSuccess) return TP_EHIP;
  EpiStore<T> epi2{static_cast<T*>(Z), h, T_, h};
  return hip_status(gemm_any<T, KMAJOR, MNMAJOR>(problem(T_, h, f, H, f, W2, nullptr, h), epi2, st));
}

template <class T>
int mlp_bwd_impl(const tp_mlp_desc& d, int f, const void* dOut, uint32_t thr, float scale, uint64_t seed,
                 const void* X, const void* W1, const void* Wu, const void* W2, const void* saved, const void* H,
                 void* dY, float* db2, void* dA, float* dW1, float* db1, float* dW2, void* dX, hipStream_t st) {
  const int T_ = (int)d.tokens, h = (int)d.h;
  const int64_t Tf = (int64_t)T_ * f;
  hipError_t e = hipSuccess;
  // a4: dropout backward (or a copy when dY is requested with p = 0)
  const void* dYp = dOut;
  if (dY) {
    if ((e = dropout_bwd<T>((int64_t)T_ * h, dOut, thr, scale, seed, dY, st)) != hipSuccess) return TP_EHIP;
    dYp = dY;
  }
  if (db2 && (e = colsum<T>(T_, h, dYp, db2, st)) != hipSuccess) return TP_EHIP;
  // a5: dH = dY W2^T with the activation backward fused, and dW2_i = H_i^T dY
  // ([f, h], K = tokens), independent of it: one paired launch for bf16 shards
  {
    const GemmProblem ph = problem(T_, f, h, dYp, h, W2, nullptr, h);
    const GemmProblem pw = problem(f, h, T_, H, f, dYp, nullptr, h);
    EpiStore<float> ew{dW2, h, f, h};
    auto run = [&](const auto& eh) -> hipError_t {
      if constexpr (std::is_same_v<T, float>) {
        hipError_t r = gemm_any<T, KMAJOR, KMAJOR>(ph, eh, st);
        return r != hipSuccess ? r : gemm_any<T, MNMAJOR, MNMAJOR>(pw, ew, st);
      } else {
        return gemm_bf16_pair<KMAJOR, KMAJOR, MNMAJOR, MNMAJOR>(ph, eh, pw, ew, st);
      }
    };
    if (d.act == TP_GELU) {
      e = run(EpiGeluBwd<T>{static_cast<const T*>(saved), static_cast<T*>(dA), f, T_, f});
    } else {
      const T* G = static_cast<const T*>(saved);
      T* dG = static_cast<T*>(dA);
      e = run(EpiSwigluBwd<T>{G, G + Tf, dG, dG + Tf, f, T_, f});
    }
  }
  if (e != hipSuccess) return TP_EHIP;
  if (db1 && (e = colsum<T>(T_, f, dA, db1, st)) != hipSuccess) return TP_EHIP;
  // a6: dW1_i = X^T dA_i  ([h, f], K = tokens); SwiGLU: dWg_i and dWu_i share the X^T tile.
  // a6: dX_i = dA_i W1_i^T  (SwiGLU: dG_i Wg_i^T + dU_i Wu_i^T, two K segments into one accumulator).
  // The two are independent; bf16 shards run them as one paired launch.
  GemmProblem pw = d.act == TP_GELU ? problem(h, f, T_, X, h, dA, nullptr, f)
                                    : problem(h, f, T_, X, h, dA, static_cast<const T*>(dA) + Tf, f);
  GemmProblem px = problem(T_, h, f, dA, f, W1, nullptr, f);
  if (d.act == TP_SWIGLU) {
    px.nseg = 2;
    px.K[1] = f;
    px.A[1] = reinterpret_cast<const uint16_t*>(static_cast<const T*>(dA) + Tf);
    px.B[1][0] = static_cast<const uint16_t*>(Wu);
  }
  EpiStore<T> ex{static_cast<T*>(dX), h, T_, h};
  if (d.act == TP_GELU) {
    EpiStore<float> ew{dW1, f, h, f};
    if constexpr (std::is_same_v<T, float>) {
      if ((e = gemm_any<T, MNMAJOR, MNMAJOR>(pw, ew, st)) != hipSuccess) return TP_EHIP;
      e = gemm_any<T, KMAJOR, KMAJOR>(px, ex, st);
    } else {
      e = gemm_bf16_pair<MNMAJOR, MNMAJOR, KMAJOR, KMAJOR>(pw, ew, px, ex, st);
    }
  } else {
    EpiStore2<float> ew{dW1, dW1 + (int64_t)h * f, f, h, f};
    if constexpr (std::is_same_v<T, float>) {
      if ((e = gemm_any<T, MNMAJOR, MNMAJOR>(pw, ew, st)) != hipSuccess) return TP_EHIP;
      e = gemm_any<T, KMAJOR, KMAJOR>(px, ex, st);
    } else {
      e = gemm_bf16_pair<MNMAJOR, MNMAJOR, KMAJOR, KMAJOR>(pw, ew, px, ex, st);
    }
  }
  return hip_status(e);
}

// The matrix-core kernels address each operand through a buffer resource with
// 32-bit byte offsets; every operand must stay below 2 GiB.
bool buffer_ok(int64_t elems, int64_t elem_bytes) { return elems * elem_bytes < ((int64_t)1 << 31); }

// This rank's intermediate columns: contiguous blocks of `unit` columns,
// dealt out in rank order as evenly as whole blocks allow (the first
// (h_ffn/unit) % t ranks take one block more); an even split when t divides
// h_ffn/unit.
void mlp_cols(int64_t h_ffn, int t, int rank, int unit, int64_t* f, int64_t* col0) {
  const int64_t u = h_ffn / unit, base = u / t, extra = u % t;
  *f = unit * (base + (rank < extra ? 1 : 0));
  *col0 = unit * (rank * base + (rank < extra ? rank : extra));
}

int validate_mlp(const tp_mlp_desc* d, bool* bf16, int64_t* f) {
  if (!d) return TP_EINVAL;
  if (d->dtype != TP_F32 && d->dtype != TP_BF16) return TP_EDTYPE;
  if (d->act != TP_GELU && d->act != TP_SWIGLU) return TP_EDTYPE;
  if (d->t < 1 || d->rank < 0 || d->rank >= d->t) return TP_EINVAL;
  if (!fits_int(d->tokens) || !fits_int(d->h) || !fits_int(d->h_ffn)) return TP_EINVAL;
  *bf16 = d->dtype == TP_BF16;
  const int vec = *bf16 ? 8 : 4;
  if (d->h % vec || d->h_ffn % vec) return TP_EALIGN;
  int64_t col0;
  mlp_cols(d->h_ffn, d->t, d->rank, vec, f, &col0);
  if (*bf16 && (!buffer_ok(d->tokens * d->h, 2) || !buffer_ok(d->tokens * *f, 2) || !buffer_ok(d->h * *f, 2)))
    return TP_EUNSUPPORTED;
  return TP_OK;
}

// This rank's heads: q query heads from q0 and kv KV heads from kv0.  Whole
// GQA groups are dealt out when n_kv >= t (the first n_kv % t ranks take one
// more); when n_kv < t each KV head is replicated on t / n_kv consecutive
// ranks that split its query heads evenly.
int attn_heads(int n_q, int n_kv, int t, int rank, int* q, int* kv, int* q0, int* kv0) {
  if (n_q % n_kv) return TP_ENOTDIV;
  const int group = n_q / n_kv;
  if (n_kv >= t) {
    const int base = n_kv / t, extra = n_kv % t;
    *kv = base + (rank < extra ? 1 : 0);
    *kv0 = rank * base + (rank < extra ? rank : extra);
    *q = *kv * group;
    *q0 = *kv0 * group;
    return TP_OK;
  }
  const int r = t / n_kv;
  if (t % n_kv || group % r) return TP_ENOTDIV;
  *kv = 1;
  *kv0 = rank / r;
  *q = group / r;
  *q0 = *kv0 * group + (rank % r) * *q;
  return TP_OK;
}

// A tensor argument is present when its pointer is non-null or it holds no elements.
bool present(const void* p, int64_t n) { return p != nullptr || n == 0; }

bool ptrs_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}

}  // namespace

extern "C" {

int tp_profile_arm(void* const* events, int32_t n_events) {
  if (n_events < 0 || n_events > 64 || (n_events & 1) || (n_events && !events)) return TP_EINVAL;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return TP_EINVAL;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < n_events; ++i) g_prof.ev[i] = static_cast<hipEvent_t>(events[i]);
  g_prof.n_kernels = n_events / 2;
  g_prof.next = 0;
  g_prof.armed.store(n_events > 0, std::memory_order_release);
  return TP_OK;
}

int tp_set_options(int32_t tile, int32_t split_tail) {
  if (tile < TP_TILE_AUTO || tile > TP_TILE_TINY || (split_tail != 0 && split_tail != 1)) return TP_EINVAL;
  g_tile.store(tile, std::memory_order_relaxed);
  g_split.store(split_tail, std::memory_order_relaxed);
  return TP_OK;
}

int tp_get_options(int32_t* tile, int32_t* split_tail) {
  if (!tile || !split_tail) return TP_EINVAL;
  *tile = g_tile.load(std::memory_order_relaxed);
  *split_tail = g_split.load(std::memory_order_relaxed);
  return TP_OK;
}

const char* tp_status_string(int s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_EINVAL: return "TP_EINVAL: invalid argument";
    case TP_ENOTDIV: return "TP_ENOTDIV: size not divisible by the TP degree or head grouping";
    case TP_EDTYPE: return "TP_EDTYPE: unsupported dtype or activation";
    case TP_EALIGN: return "TP_EALIGN: pointer or width not aligned to 16 bytes";
    case TP_EHIP: return "TP_EHIP: HIP runtime error at launch";
    case TP_EUNSUPPORTED: return "TP_EUNSUPPORTED: size not implemented by the kernels";
    case TP_ENOSCRATCH: return "TP_ENOSCRATCH: the problem needs more scratch than the library's fixed device array";
    default: return "unknown status";
  }
}

int tp_mlp_shard_cols(int64_t h_ffn, int32_t t, int32_t rank, int32_t dtype, int64_t* f_i, int64_t* col0) {
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_EDTYPE;
  if (!f_i || !col0 || h_ffn < 0 || t < 1 || rank < 0 || rank >= t) return TP_EINVAL;
  const int vec = dtype == TP_BF16 ? 8 : 4;
  if (h_ffn % vec) return TP_EALIGN;
  mlp_cols(h_ffn, t, rank, vec, f_i, col0);
  return TP_OK;
}

int tp_attn_shard_heads(int32_t n_q, int32_t n_kv, int32_t t, int32_t rank, int32_t* q_i, int32_t* kv_i,
                        int32_t* q0, int32_t* kv0) {
  if (!q_i || !kv_i || !q0 || !kv0 || n_q < 1 || n_kv < 1 || t < 1 || rank < 0 || rank >= t) return TP_EINVAL;
  int q, kv, a, b;
  if (int rc = attn_heads(n_q, n_kv, t, rank, &q, &kv, &a, &b)) return rc;
  *q_i = q;
  *kv_i = kv;
  *q0 = a;
  *kv0 = b;
  return TP_OK;
}

int tp_comm_bytes(int64_t tokens, int64_t h, int32_t t, int32_t delta, tp_comm* out) {
  if (!out || tokens < 0 || h < 0 || t < 1 || delta < 1) return TP_EINVAL;
  const uint64_t payload = (uint64_t)tokens * (uint64_t)h * (uint64_t)delta;
  out->n_allreduce_fwd = 2;
  out->n_allreduce_bwd = 2;
  out->payload_bytes = payload;
  out->ring_bytes_per_rank = 2.0 * (double)(t - 1) / (double)t * (double)payload;
  out->layer_payload_bytes = 4 * payload;
  out->layer_ring_bytes_per_rank = 4.0 * out->ring_bytes_per_rank;
  return TP_OK;
}

int tp_mlp_shard_fwd(const tp_mlp_desc* desc, const void* X, const void* W1_i, const void* Wu_i, const void* b1_i,
                     const void* W2_i, void* saved_i, void* H_i, void* Z_i, void* stream) {
  bool bf16 = false;
  int64_t f = 0;
  int rc = validate_mlp(desc, &bf16, &f);
  if (rc) return rc;
  {
    const int64_t T_ = desc->tokens, h = desc->h, ns = desc->act == TP_GELU ? 1 : 2;
    if (!present(X, T_ * h) || !present(W1_i, h * f) || !present(W2_i, f * h) || !present(saved_i, ns * T_ * f) ||
        !present(H_i, T_ * f) || !present(Z_i, T_ * h) || (desc->act == TP_SWIGLU && !present(Wu_i, h * f)))
      return TP_EINVAL;
  }
  if (desc->act == TP_GELU ? (Wu_i != nullptr) : (b1_i != nullptr)) return TP_EINVAL;
  if (!ptrs_aligned({X, W1_i, Wu_i, b1_i, W2_i, saved_i, H_i, Z_i})) return TP_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return bf16 ? mlp_fwd_impl<uint16_t>(*desc, (int)f, X, W1_i, Wu_i, b1_i, W2_i, saved_i, H_i, Z_i, st)
              : mlp_fwd_impl<float>(*desc, (int)f, X, W1_i, Wu_i, b1_i, W2_i, saved_i, H_i, Z_i, st);
}

int tp_mlp_shard_bwd(const tp_mlp_desc* desc, const void* dOut, float p_drop, uint64_t seed, const void* X,
                     const void* W1_i, const void* Wu_i, const void* W2_i, const void* saved_i, const void* H_i,
                     void* dY, float* db2, void* dA_i, float* dW1_i, float* db1_i, float* dW2_i, void* dX_i,
                     void* stream) {
  bool bf16 = false;
  int64_t f = 0;
  int rc = validate_mlp(desc, &bf16, &f);
  if (rc) return rc;
  uint32_t thr = 0;
  float scale = 1.0f;
  if ((rc = check_dropout(p_drop, &thr, &scale))) return rc;
  {
    const int64_t T_ = desc->tokens, h = desc->h, ns = desc->act == TP_GELU ? 1 : 2;
    if (!present(dOut, T_ * h) || !present(X, T_ * h) || !present(W1_i, h * f) || !present(W2_i, f * h) ||
        !present(saved_i, ns * T_ * f) || !present(H_i, T_ * f) || !present(dA_i, ns * T_ * f) ||
        !present(dW1_i, ns * h * f) || !present(dW2_i, f * h) || !present(dX_i, T_ * h) ||
        (desc->act == TP_SWIGLU && !present(Wu_i, h * f)))
      return TP_EINVAL;
  }
  if (desc->act == TP_GELU ? (Wu_i != nullptr) : (db1_i != nullptr)) return TP_EINVAL;
  if (thr != 0 && !dY) return TP_EINVAL;
  if (!ptrs_aligned({dOut, X, W1_i, Wu_i, W2_i, saved_i, H_i, dY, db2, dA_i, dW1_i, db1_i, dW2_i, dX_i}))
    return TP_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return bf16 ? mlp_bwd_impl<uint16_t>(*desc, (int)f, dOut, thr, scale, seed, X, W1_i, Wu_i, W2_i, saved_i, H_i,
                                       dY, db2, dA_i, dW1_i, db1_i, dW2_i, dX_i, st)
              : mlp_bwd_impl<float>(*desc, (int)f, dOut, thr, scale, seed, X, W1_i, Wu_i, W2_i, saved_i, H_i, dY,
                                    db2, dA_i, dW1_i, db1_i, dW2_i, dX_i, st);
}

// Descriptor checks shared by the attention entry points.
int check_attn_desc(const tp_attn_desc* d) {
  if (!d) return TP_EINVAL;
  if (d->dtype != TP_BF16) return TP_EDTYPE;
  if (d->b < 0 || d->s < 0 || d->h < 0 || d->n_q < 1 || d->n_kv < 1 || d->d < 1 || d->t < 1 || d->rank < 0 ||
      d->rank >= d->t)
    return TP_EINVAL;
  int q, kv, q0, kv0;
  if (int rc = attn_heads(d->n_q, d->n_kv, d->t, d->rank, &q, &kv, &q0, &kv0)) return rc;
  if (d->d != 64 && d->d != 128) return TP_EUNSUPPORTED;
  if (!fits_int(d->b * d->s) || !fits_int(d->h)) return TP_EINVAL;
  // the attention kernels' tile loads form row offsets with 24-bit multiplies
  if (d->s >= (1 << 24) || (int64_t)(q + 2 * kv) * d->d * 2 >= (1 << 24)) return TP_EUNSUPPORTED;
  return TP_OK;
}

// This rank's query and KV head counts (the descriptor has been checked).
void local_heads(const tp_attn_desc* d, int* q, int* kv) {
  int q0, kv0;
  attn_heads(d->n_q, d->n_kv, d->t, d->rank, q, kv, &q0, &kv0);
}

// Query heads per work-group of the attention kernels: four, two or one, so
// that the heads of a work-group share one KV head.
int heads_per_wg(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }

int tp_attn_shard_fwd(const tp_attn_desc* d, const void* X, const void* Wqkv_i, const void* Wo_i, void* QKV_i,
                      void* O_i, float* lse_i, void* Z_i, void* stream) {
  if (int rc = check_attn_desc(d)) return rc;
  int q, kv;
  local_heads(d, &q, &kv);
  {
    const int64_t T_ = d->b * d->s, nq = (int64_t)q * d->d, nkv = (int64_t)kv * d->d;
    if (!present(X, T_ * d->h) || !present(Wqkv_i, d->h * (nq + 2 * nkv)) || !present(Wo_i, nq * d->h) ||
        !present(QKV_i, T_ * (nq + 2 * nkv)) || !present(O_i, T_ * nq) || !present(Z_i, T_ * d->h))
      return TP_EINVAL;
  }
  if (d->h % 8) return TP_EALIGN;
  if (!ptrs_aligned({X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i})) return TP_EALIGN;
  {
    const int64_t T_ = d->b * d->s, nqkv = (int64_t)(q + 2 * kv) * d->d;
    if (!buffer_ok(T_ * d->h, 2) || !buffer_ok(T_ * nqkv, 2) || !buffer_ok(d->h * nqkv, 2)) return TP_EUNSUPPORTED;
  }
  const int D = d->d;
  const int T_ = (int)(d->b * d->s), h = (int)d->h;
  const int nqkv = (q + 2 * kv) * D;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // QKV_i = X Wqkv_i
  EpiStore<uint16_t> e1{static_cast<uint16_t*>(QKV_i), nqkv, T_, nqkv};
  if (gemm_bf16<KMAJOR, MNMAJOR>(problem(T_, nqkv, h, X, h, Wqkv_i, nullptr, nqkv), e1, st) != hipSuccess)
    return TP_EHIP;
  // local heads' attention
  attn::AttnArgs a{};
  a.qkv = static_cast<const uint16_t*>(QKV_i);
  a.o = static_cast<uint16_t*>(O_i);
  a.lse = lse_i;
  a.ld_qkv = nqkv;
  a.ld_o = (int64_t)q * D;
  a.b = (int)d->b;
  a.s = (int)d->s;
  a.q = q;
  a.kv = kv;
  a.hg = heads_per_wg(q / kv);
  a.causal = d->causal ? 1 : 0;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  // the heaviest query blocks of a launch that leaves slots empty run as two
  // halves whose softmax state goes to Z_i's memory (written only by the
  // output projection below)
  a.paired = split_tail_enabled() && attn_fwd_paired(a.s, a.causal, a.b, a.q, a.kv, a.hg) ? 1 : 0;
  a.split = split_tail_enabled() && !a.paired ? attn_fwd_split(a.s, a.causal, a.b, a.q, a.kv, a.hg) : 0;
  if (attn_fwd_part_floats(a.b, a.q, a.kv, a.hg, a.split, D) * 4 > (int64_t)T_ * h * 2) a.split = 0;
  a.part = static_cast<float*>(Z_i);
  hipError_t e;
  {
    Probe pr(st);
    e = D == 128 ? launch_attn_fwd<128>(a, st) : launch_attn_fwd<64>(a, st);
  }
  if (e != hipSuccess) return TP_EHIP;
  // Z_i = O_i Wo_i
  EpiStore<uint16_t> e2{static_cast<uint16_t*>(Z_i), h, T_, h};
  return hip_status(gemm_bf16<KMAJOR, MNMAJOR>(problem(T_, h, q * D, O_i, q * D, Wo_i, nullptr, h), e2, st));
}

}  // extern "C"

namespace {

// Argument checks of the attention backward, stats_i aside.
int check_attn_bwd(const tp_attn_desc* d, const void* dZ, const void* X, const void* Wqkv_i, const void* Wo_i,
                   const void* QKV_i, const void* O_i, const float* lse_i, const void* dO_i, const void* dQKV_i,
                   const float* dWqkv_i, const float* dWo_i, const void* dX_i) {
  if (int rc = check_attn_desc(d)) return rc;
  int q, kv;
  local_heads(d, &q, &kv);
  const int64_t T64 = d->b * d->s, nq64 = (int64_t)q * d->d;
  const int64_t nqkv64 = (int64_t)(q + 2 * kv) * d->d, rows64 = d->b * (int64_t)q * d->s;
  if (!present(dZ, T64 * d->h) || !present(X, T64 * d->h) || !present(Wqkv_i, d->h * nqkv64) ||
      !present(Wo_i, nq64 * d->h) || !present(QKV_i, T64 * nqkv64) || !present(O_i, T64 * nq64) ||
      !present(lse_i, rows64) || !present(dO_i, T64 * nq64) || !present(dQKV_i, T64 * nqkv64) ||
      !present(dWqkv_i, d->h * nqkv64) || !present(dWo_i, nq64 * d->h) || !present(dX_i, T64 * d->h))
    return TP_EINVAL;
  if (d->h % 8) return TP_EALIGN;
  if (!ptrs_aligned({dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, dQKV_i, dWqkv_i, dWo_i, dX_i})) return TP_EALIGN;
  if (!buffer_ok(T64 * d->h, 2) || !buffer_ok(T64 * nqkv64, 2) || !buffer_ok(d->h * nqkv64, 2) ||
      !buffer_ok(2 * rows64, 4))
    return TP_EUNSUPPORTED;
  return TP_OK;
}

// Fp32 floats of the per-row statistics the attention backward keeps between its kernels.
int64_t attn_bwd_stats_floats(const tp_attn_desc* d) {
  int q, kv;
  local_heads(d, &q, &kv);
  return 2 * d->b * (int64_t)q * d->s;
}

// The attention backward's launches, arguments checked; stats_i holds
// attn_bwd_stats_floats() floats.
int attn_bwd_impl(const tp_attn_desc* d, const void* dZ, const void* X, const void* Wqkv_i, const void* Wo_i,
                  const void* QKV_i, const void* O_i, const float* lse_i, void* dO_i, float* stats_i, void* dQKV_i,
                  float* dWqkv_i, float* dWo_i, void* dX_i, void* stream) {
  int q, kv;
  local_heads(d, &q, &kv);
  const int64_t T64 = d->b * d->s;
  const int64_t nqkv64 = (int64_t)(q + 2 * kv) * d->d;
  const int D = d->d;
  const int T_ = (int)T64, h = (int)d->h, nq = q * D, nqkv = (q + 2 * kv) * D;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // dO_i = dZ Wo_i^T (Wo_i [q d, h] is K-contiguous for this product) and,
  // independent of it, dWo_i = O_i^T dZ: one paired launch
  EpiStore<uint16_t> e1{static_cast<uint16_t*>(dO_i), nq, T_, nq};
  EpiStore<float> e2{dWo_i, h, nq, h};
  if (gemm_bf16_pair<KMAJOR, KMAJOR, MNMAJOR, MNMAJOR>(problem(T_, nq, h, dZ, h, Wo_i, nullptr, h), e1,
                                                       problem(nq, h, T_, O_i, nq, dZ, nullptr, h), e2,
                                                       st) != hipSuccess)
    return TP_EHIP;
  // the core: row statistics, dK/dV, dQ
  attnb::BwdArgs a{};
  a.qkv = static_cast<const uint16_t*>(QKV_i);
  a.o = static_cast<const uint16_t*>(O_i);
  a.dO = static_cast<const uint16_t*>(dO_i);
  a.lse = lse_i;
  a.stats = stats_i;
  a.dqkv = static_cast<uint16_t*>(dQKV_i);
  a.ld_qkv = nqkv;
  a.ld_o = nq;
  a.b = (int)d->b;
  a.s = (int)d->s;
  a.q = q;
  a.kv = kv;
  a.causal = d->causal ? 1 : 0;
  a.scale = (float)(1.0 / std::sqrt((double)D));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  // dK/dV's heaviest key blocks run as two halves whose fp32 sums go to
  // dWqkv_i's memory, written only by the last GEMM below
  a.split = split_tail_enabled() ? attn_bwd_dkv_split(a.s, a.causal) : 0;
  if (a.split > 0) {  // as many as dWqkv_i's memory holds
    const int64_t per_block = attn_bwd_dkv_part_floats(a.b, a.kv, 1, D);
    const int64_t fits = per_block > 0 ? d->h * nqkv64 / per_block : 0;
    if (fits < a.split) a.split = (int)fits;
  }
  a.dkv_part = dWqkv_i;
  const int hg = heads_per_wg(q / kv);
  // dQ's heaviest query blocks likewise, their halves' sums in dX_i's memory
  // (written only by the last GEMM below)
  // dK/dV hands its dS tiles to dQ (no recompute of the scores there) where
  // they fit in dX_i's memory and the part of dWqkv_i's after the dK/dV
  // halves, both written only by the last GEMM below
  a.ds_path = 0;
  if (split_tail_enabled() && a.causal) {
    const int64_t nqt = (a.s + 31) / 32;
    const int64_t tiles = (int64_t)a.b * a.q * (nqt * (nqt + 1) / 2);
    const int64_t cap_a = T64 * d->h * 2 / 2048;
    const int64_t part_bytes = a.split > 0 ? attn_bwd_dkv_part_floats(a.b, a.kv, a.split, D) * 4 : 0;
    const int64_t b_off = (part_bytes + 2047) / 2048 * 2048;
    const int64_t cap_b = d->h * nqkv64 * 4 > b_off ? (d->h * nqkv64 * 4 - b_off) / 2048 : 0;
    if (tiles > 0 && tiles <= cap_a + cap_b) {
      a.ds_path = 1;
      a.ds_a = static_cast<uint8_t*>(dX_i);
      a.ds_t0 = tiles < cap_a ? tiles : cap_a;
      a.ds_b = reinterpret_cast<uint8_t*>(dWqkv_i) + b_off;
    }
  }
  a.dq_split = split_tail_enabled() && !a.ds_path ? attn_bwd_dq_split(a.s, a.causal, a.b, a.q, a.kv, hg) : 0;
  if (attn_bwd_dq_part_floats(a.b, a.q, a.kv, hg, a.dq_split, D) * 4 > T64 * d->h * 2) a.dq_split = 0;
  a.dq_part = static_cast<float*>(dX_i);
  hipError_t e;
  {
    Probe pr(st);
    e = D == 128 ? launch_attn_bwd_stats<128>(a, st) : launch_attn_bwd_stats<64>(a, st);
  }
  if (e != hipSuccess) return TP_EHIP;
  {
    Probe pr(st);
    e = D == 128 ? launch_attn_bwd_dkv<128>(a, st) : launch_attn_bwd_dkv<64>(a, st);
  }
  if (e != hipSuccess) return TP_EHIP;
  {
    Probe pr(st);
    e = D == 128 ? launch_attn_bwd_dq<128>(a, hg, st) : launch_attn_bwd_dq<64>(a, hg, st);
  }
  if (e != hipSuccess) return TP_EHIP;
  // dWqkv_i = X^T dQKV_i (K = tokens) and dX_i = dQKV_i Wqkv_i^T (Wqkv_i [h, (q+2kv) d]
  // is K-contiguous for this product; K = (q+2kv) d): one paired launch, longer K first
  EpiStore<float> e3{dWqkv_i, nqkv, h, nqkv};
  EpiStore<uint16_t> e4{static_cast<uint16_t*>(dX_i), h, T_, h};
  return hip_status(gemm_bf16_pair<MNMAJOR, MNMAJOR, KMAJOR, KMAJOR>(
      problem(h, nqkv, T_, X, h, dQKV_i, nullptr, nqkv), e3,
      problem(T_, h, nqkv, dQKV_i, nqkv, Wqkv_i, nullptr, nqkv), e4, st));
}

}  // namespace

extern "C" {

int tp_attn_shard_bwd(const tp_attn_desc* d, const void* dZ, const void* X, const void* Wqkv_i, const void* Wo_i,
                      const void* QKV_i, const void* O_i, const float* lse_i, void* dO_i, float* stats_i,
                      void* dQKV_i, float* dWqkv_i, float* dWo_i, void* dX_i, void* stream) {
  if (int rc = check_attn_bwd(d, dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, dQKV_i, dWqkv_i, dWo_i, dX_i))
    return rc;
  if (!present(stats_i, attn_bwd_stats_floats(d))) return TP_EINVAL;
  if (!aligned16(stats_i)) return TP_EALIGN;
  return attn_bwd_impl(d, dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, stats_i, dQKV_i, dWqkv_i, dWo_i, dX_i,
                       stream);
}

}  // extern "C"

// Device memory of tp_attn_shard_bwd_noalloc: the per-row statistics
// ({lse * log2(e), rowsum(dO * O)} per row) that tp_attn_shard_bwd keeps in
// its caller's stats_i.  Every GPU holds its own copy for the life of the
// process; host code must use the address hipGetSymbolAddress returns for
// the current device, never the array's name.
constexpr int64_t kScratchFloats = (int64_t)1 << 20;  // 4 MiB: b * q * s up to 524288 rows
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
struct ScratchTable {
  std::mutex mu;
  float* ptr[kMaxDevices] = {};
} g_scratch;

// Device address of `scratch` on the current device, looked up once per device.
int scratch_for_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TP_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TP_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TP_EHIP;
    g_scratch.ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch.ptr[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_attn_shard_bwd_noalloc(const tp_attn_desc* d, const void* dZ, const void* X, const void* Wqkv_i,
                              const void* Wo_i, const void* QKV_i, const void* O_i, const float* lse_i, void* dO_i,
                              void* dQKV_i, float* dWqkv_i, float* dWo_i, void* dX_i, void* stream) {
  if (int rc = check_attn_bwd(d, dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, dQKV_i, dWqkv_i, dWo_i, dX_i))
    return rc;
  if (attn_bwd_stats_floats(d) > kScratchFloats) return TP_ENOSCRATCH;
  float* stats = nullptr;
  if (int rc = scratch_for_current_device(&stats)) return rc;
  return attn_bwd_impl(d, dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, stats, dQKV_i, dWqkv_i, dWo_i, dX_i, stream);
}

}  // extern "C"

namespace {

// Rows [row0, row0 + nrows) of residual + Dropout(sum_i P_i + bias) over full
// [rows_total, cols] partials, written to out [nrows, cols]; the residual, if
// any, is [nrows, cols].  Shared by the all-reduce and the reduce-scatter.
int sum_rows(int64_t rows_total, int64_t row0, int64_t nrows, int64_t cols, int32_t t, int32_t dtype,
             const void* const* partials, const void* bias, float p_drop, uint64_t seed, const void* residual,
             void* out, void* stream) {
  uint32_t thr = 0;
  float scale = 1.0f;
  int rc = check_dropout(p_drop, &thr, &scale);
  if (rc) return rc;
  const int vec = dtype == TP_BF16 ? 8 : 4;
  const int esz = dtype == TP_BF16 ? 2 : 4;
  if (cols % vec) return TP_EALIGN;
  PartialPtrs P{};
  for (int i = 0; i < t; ++i) {
    if (!present(partials[i], rows_total * cols)) return TP_EINVAL;
    if (!aligned16(partials[i])) return TP_EALIGN;
    P.p[i] = partials[i] ? static_cast<const uint8_t*>(partials[i]) + row0 * cols * esz : nullptr;
  }
  if (!ptrs_aligned({bias, residual, out})) return TP_EALIGN;
  const int64_t nv = nrows * cols / vec;
  if (nv == 0) return TP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t idx0 = (uint64_t)(row0 * cols);
  Probe pr(st);
  if (dtype == TP_BF16)
    tp_launch(sum_partials_kernel<uint16_t>, dim3(grid_for(nv)), dim3(256), 0, st, nv, cols, t, P,
              static_cast<const uint16_t*>(bias), thr, scale, seed, idx0,
              static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out));
  else
    tp_launch(sum_partials_kernel<float>, dim3(grid_for(nv)), dim3(256), 0, st, nv, cols, t, P,
              static_cast<const float*>(bias), thr, scale, seed, idx0, static_cast<const float*>(residual),
              static_cast<float*>(out));
  return hip_status(hipGetLastError());
}

// Largest row the fused norm keeps in registers: 16 vectors per thread of 256.
constexpr int64_t kNormMaxVecs = 16 * 256;

template <class T, int NV>
void launch_sum_norm(int64_t nrows, int64_t cols, int t, const PartialPtrs& P, const void* bias, uint32_t thr,
                     float scale, uint64_t seed, uint64_t idx0, const void* residual, int layer, const void* gamma,
                     const void* beta, float eps, void* out, void* normed, hipStream_t st) {
  tp_launch((sum_norm_kernel<T, NV>), dim3((unsigned)nrows), dim3(256), 0, st, cols, t, P,
            static_cast<const T*>(bias), thr, scale, seed, idx0, static_cast<const T*>(residual), layer,
            static_cast<const T*>(gamma), static_cast<const T*>(beta), eps, static_cast<T*>(out),
            static_cast<T*>(normed));
}

template <class T>
void sum_norm_dispatch(int64_t nrows, int64_t cols, int t, const PartialPtrs& P, const void* bias, uint32_t thr,
                       float scale, uint64_t seed, uint64_t idx0, const void* residual, int layer, const void* gamma,
                       const void* beta, float eps, void* out, void* normed, hipStream_t st) {
  const int64_t per = (cols / Vec<T>::N + 255) / 256;
  if (per <= 1)
    launch_sum_norm<T, 1>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps, out,
                          normed, st);
  else if (per <= 2)
    launch_sum_norm<T, 2>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps, out,
                          normed, st);
  else if (per <= 4)
    launch_sum_norm<T, 4>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps, out,
                          normed, st);
  else if (per <= 8)
    launch_sum_norm<T, 8>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps, out,
                          normed, st);
  else
    launch_sum_norm<T, 16>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps, out,
                           normed, st);
}

// Rows [row0, row0 + nrows) of the block output and their norm (shared by the
// fused all-reduce + norm and the reduce-scatter + norm).
int sum_rows_norm(int64_t rows_total, int64_t row0, int64_t nrows, int64_t cols, int32_t t, int32_t dtype,
                  const void* const* partials, const void* bias, float p_drop, uint64_t seed, const void* residual,
                  int32_t norm, const void* gamma, const void* beta, float eps, void* out, void* normed,
                  void* stream) {
  if (norm != TP_NORM_RMS && norm != TP_NORM_LAYER) return TP_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return TP_EINVAL;
  if (norm == TP_NORM_RMS && beta) return TP_EINVAL;
  uint32_t thr = 0;
  float scale = 1.0f;
  if (int rc = check_dropout(p_drop, &thr, &scale)) return rc;
  const int vec = dtype == TP_BF16 ? 8 : 4;
  const int esz = dtype == TP_BF16 ? 2 : 4;
  if (cols % vec) return TP_EALIGN;
  if (cols / vec > kNormMaxVecs) return TP_EUNSUPPORTED;
  if (!present(out, nrows * cols) || !present(normed, nrows * cols)) return TP_EINVAL;
  PartialPtrs P{};
  for (int i = 0; i < t; ++i) {
    if (!present(partials[i], rows_total * cols)) return TP_EINVAL;
    if (!aligned16(partials[i])) return TP_EALIGN;
    P.p[i] = partials[i] ? static_cast<const uint8_t*>(partials[i]) + row0 * cols * esz : nullptr;
  }
  if (!ptrs_aligned({bias, residual, gamma, beta, out, normed})) return TP_EALIGN;
  if (nrows == 0 || cols == 0) return TP_OK;
  if (nrows > INT32_MAX) return TP_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t idx0 = (uint64_t)(row0 * cols);
  const int layer = norm == TP_NORM_LAYER ? 1 : 0;
  Probe pr(st);
  if (dtype == TP_BF16)
    sum_norm_dispatch<uint16_t>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps,
                                out, normed, st);
  else
    sum_norm_dispatch<float>(nrows, cols, t, P, bias, thr, scale, seed, idx0, residual, layer, gamma, beta, eps, out,
                             normed, st);
  return hip_status(hipGetLastError());
}

int check_sum_args(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials) {
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_EDTYPE;
  if (rows < 0 || cols < 0 || t < 1 || !partials) return TP_EINVAL;
  if (t > MAX_PARTIALS) return TP_EUNSUPPORTED;
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_sum_partials(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials,
                    const void* bias, float p_drop, uint64_t seed, void* out, void* stream) {
  return tp_sum_partials_residual(rows, cols, t, dtype, partials, bias, p_drop, seed, nullptr, out, stream);
}

int tp_sum_partials_residual(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials,
                             const void* bias, float p_drop, uint64_t seed, const void* residual, void* out,
                             void* stream) {
  if (int rc = check_sum_args(rows, cols, t, dtype, partials)) return rc;
  if (!present(out, rows * cols)) return TP_EINVAL;
  return sum_rows(rows, 0, rows, cols, t, dtype, partials, bias, p_drop, seed, residual, out, stream);
}

int tp_reduce_scatter(int64_t rows, int64_t cols, int32_t t, int32_t rank, int32_t dtype,
                      const void* const* partials, const void* bias, float p_drop, uint64_t seed,
                      const void* residual_r, void* out_r, void* stream) {
  if (int rc = check_sum_args(rows, cols, t, dtype, partials)) return rc;
  if (rank < 0 || rank >= t) return TP_EINVAL;
  if (rows % t) return TP_ENOTDIV;
  const int64_t n = rows / t;
  if (!present(out_r, n * cols)) return TP_EINVAL;
  return sum_rows(rows, rank * n, n, cols, t, dtype, partials, bias, p_drop, seed, residual_r, out_r, stream);
}

int tp_sum_partials_norm(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials,
                         const void* bias, float p_drop, uint64_t seed, const void* residual, int32_t norm,
                         const void* gamma, const void* beta, float eps, void* out, void* normed, void* stream) {
  if (int rc = check_sum_args(rows, cols, t, dtype, partials)) return rc;
  return sum_rows_norm(rows, 0, rows, cols, t, dtype, partials, bias, p_drop, seed, residual, norm, gamma, beta, eps,
                       out, normed, stream);
}

int tp_reduce_scatter_norm(int64_t rows, int64_t cols, int32_t t, int32_t rank, int32_t dtype,
                           const void* const* partials, const void* bias, float p_drop, uint64_t seed,
                           const void* residual_r, int32_t norm, const void* gamma, const void* beta, float eps,
                           void* out_r, void* normed_r, void* stream) {
  if (int rc = check_sum_args(rows, cols, t, dtype, partials)) return rc;
  if (rank < 0 || rank >= t) return TP_EINVAL;
  if (rows % t) return TP_ENOTDIV;
  const int64_t n = rows / t;
  return sum_rows_norm(rows, rank * n, n, cols, t, dtype, partials, bias, p_drop, seed, residual_r, norm, gamma, beta,
                       eps, out_r, normed_r, stream);
}

int tp_all_gather(int64_t rows_per_rank, int64_t cols, int32_t t, int32_t dtype, const void* const* slices,
                  void* out, void* stream) {
  if (dtype != TP_F32 && dtype != TP_BF16) return TP_EDTYPE;
  if (rows_per_rank < 0 || cols < 0 || t < 1 || !slices) return TP_EINVAL;
  if (t > MAX_PARTIALS) return TP_EUNSUPPORTED;
  const int esz = dtype == TP_BF16 ? 2 : 4;
  if ((cols * esz) % 16) return TP_EALIGN;
  const int64_t n = rows_per_rank * cols;
  if (!present(out, n * t)) return TP_EINVAL;
  PartialPtrs S{};
  for (int i = 0; i < t; ++i) {
    if (!present(slices[i], n)) return TP_EINVAL;
    if (!aligned16(slices[i])) return TP_EALIGN;
    S.p[i] = slices[i];
  }
  if (!aligned16(out)) return TP_EALIGN;
  const int64_t nv = n * esz / 16;
  if (nv == 0) return TP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Probe pr(st);
  tp_launch(gather_kernel, dim3(grid_for(nv * t)), dim3(256), 0, st, nv, t, S, static_cast<u32x4*>(out));
  return hip_status(hipGetLastError());
}

}  // extern "C"
