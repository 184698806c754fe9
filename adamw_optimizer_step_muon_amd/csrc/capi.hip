// Exported C ABI (include/muon_adamw.h): argument checks, routing, workspace layout
// and the launch sequence of one optimizer step.  Host code only; the arithmetic is
// in the kernels of adamw.hip, muon_elementwise.hip and ns_gemm.hip.
#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "muon_adamw.h"
#include "ma_internal.h"

namespace ma {

// the Gram-space route's effective mode for these hyperparameters (defined below)
bool gram_space_range_ok(const ma_muon_hparams* hp);
int32_t gs_mode(const ma_muon_hparams* hp);
namespace {

// Workspace of ma_muon_step_static: a file-scope device array, one copy per GPU, kept
// until the process ends.  Host code never uses this name as an address (on the host it
// is only a handle); it resolves each device's copy with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MA_STATIC_WORKSPACE_BYTES];

thread_local std::string g_last_error;

ma_status fail(ma_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ma_status hip_fail(hipError_t e, const char* what) {
  return fail(MA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The quintic of the newton_schulz listing ("Optimizers: AdamW, Muon and the
// distributed optimizer", section "Muon: orthogonalising the update").
constexpr NsCoeffs kQuintic{3.4445f, -4.7750f, 2.0315f};

bool finite(float x) { return std::isfinite(x); }

struct Range {
  uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

// Largest sizes the kernels' index arithmetic is written for.
constexpr int64_t kMaxSide = int64_t(1) << 20;   // m_pad, n_pad
// (with room for the GEMM launch rounding each group's block count up to a multiple of 8
// in int arithmetic)
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 4096;

ma_status check_hparams(const ma_muon_hparams* hp) {
  if (!hp) return fail(MA_ERR_INVALID_ARG, "hparams is NULL");
  if (!finite(hp->lr) || !finite(hp->momentum) || !finite(hp->weight_decay) ||
      !finite(hp->ns_eps))
    return fail(MA_ERR_INVALID_ARG, "non-finite Muon hyperparameter");
  if (hp->ns_steps < 0 || hp->ns_steps > MA_MAX_NS_STEPS)
    return fail(MA_ERR_INVALID_ARG, "ns_steps %d outside [0, %d]", hp->ns_steps, MA_MAX_NS_STEPS);
  if (hp->scale_mode != 0 && hp->scale_mode != 1)
    return fail(MA_ERR_INVALID_ARG, "scale_mode %d is not 0 or 1", hp->scale_mode);
  if (hp->ns_mode != 0 && hp->ns_mode != 1)
    return fail(MA_ERR_INVALID_ARG, "ns_mode %d is not 0 or 1", hp->ns_mode);
  if (hp->ns_coeffs) {
    for (int i = 0; i < 3 * hp->ns_steps; ++i)
      if (!finite(hp->ns_coeffs[i])) return fail(MA_ERR_INVALID_ARG, "non-finite ns_coeffs[%d]", i);
  }
  return MA_OK;
}

NsCoeffs coeff_at(const ma_muon_hparams* hp, int it) {
  if (!hp->ns_coeffs) return kQuintic;
  return NsCoeffs{hp->ns_coeffs[3 * it], hp->ns_coeffs[3 * it + 1], hp->ns_coeffs[3 * it + 2]};
}

ma_status check_shape(int64_t K, int64_t A, int64_t B) {
  if (K < 0) return fail(MA_ERR_INVALID_ARG, "K = %lld < 0", (long long)K);
  if (K == 0) return MA_OK;
  if (A < 1 || B < 1)
    return fail(MA_ERR_INVALID_ARG, "matrix shape %lld x %lld", (long long)A, (long long)B);
  const int64_t m = A < B ? A : B, n = A < B ? B : A;
  if (round_up(m, 256) > kMaxSide || round_up(n, 256) > kMaxSide)
    return fail(MA_ERR_UNSUPPORTED, "matrix side above %lld", (long long)kMaxSide);
  // grid limits: (nblk, K) and (Bp/64, Ap/64, K) launches, K x tiles GEMM launches
  const BucketPlan p = plan_bucket(K, A, B);
  const int64_t tiles = (p.m_pad / p.tile) * (p.n_pad / p.tile);
  if (K > 65535 || K * p.nblk > kMaxBlocks || K * tiles > kMaxBlocks ||
      K * A * B / 4 / 256 > kMaxBlocks)
    return fail(MA_ERR_UNSUPPORTED, "bucket (%lld, %lld, %lld) exceeds the launch grid",
                (long long)K, (long long)A, (long long)B);
  return MA_OK;
}

ma_muon_route route_of(const BucketPlan& p, int ns_steps) {
  ma_muon_route r;
  r.transposed = p.transposed ? 1 : 0;
  r.m = static_cast<int32_t>(p.m);
  r.n = static_cast<int32_t>(p.n);
  r.ns_steps_run = ns_steps;
  r.m_pad = static_cast<int32_t>(p.m_pad);
  r.n_pad = static_cast<int32_t>(p.n_pad);
  r.ns_mode_run = (p.gram_space && ns_steps > 0) ? 1 : 0;
  return r;
}

// Buckets run in phases: consecutive buckets with the same GEMM tile (and the same
// choice of keeping X^T, which fixes the combine's operand layout), at most
// kMaxGemmGroups of them and kPhaseBytes of workspace together, share each Newton-Schulz
// launch (short Gram sides fill the chip together); each has its own workspace region.
constexpr size_t kPhaseBytes = size_t(4) << 30;

struct Phase {
  int n = 0;
  int tile = 0;
  size_t bytes = 0;
  BucketPlan plan[kMaxGemmGroups];
  size_t base[kMaxGemmGroups];
  int bucket[kMaxGemmGroups];
};

bool phase_accepts(const Phase& ph, const BucketPlan& p) {
  return ph.n > 0 && ph.n < kMaxGemmGroups && ph.tile == p.tile &&
         ph.plan[0].keeps_xt == p.keeps_xt && ph.plan[0].gram_space == p.gram_space &&
         ph.bytes + p.bytes <= kPhaseBytes;
}

void phase_add(Phase& ph, const BucketPlan& p, int bucket) {
  ph.plan[ph.n] = p;
  ph.base[ph.n] = ph.bytes;
  ph.bucket[ph.n] = bucket;
  ph.tile = p.tile;
  ph.bytes += p.bytes;  // plan sizes are multiples of 256
  ++ph.n;
}

// The buckets of a phase share its GEMM launches, so the tile that fills the chip is a
// property of the phase: a phase of 128-tile buckets (Gram sides of at least 512) whose
// 256-tiles fill the chip together, by the rule pick_tile applies to one bucket, is
// re-planned on 256-tiles, unless that would outgrow the phase's workspace or make a
// bucket keep X^T.  Measured: the 12-layer GPT's three 768-wide buckets, each faster on
// 128-tiles alone, run their shared launches 3-4 % faster on 256-tiles.
void promote(Phase& ph) {
  if (ph.tile != 128 || forced_tile()) return;
  int64_t tri = 0, comb = 0;
  for (int j = 0; j < ph.n; ++j) {
    const BucketPlan& p = ph.plan[j];
    if (p.m < kMinGram256) return;
    tri += tri_tiles_256(p.K, p.m);
    comb += comb_tiles_256(p.K, p.m, p.n);
  }
  if (!fills_256(tri, comb)) return;
  Phase q;
  for (int j = 0; j < ph.n; ++j) {
    const BucketPlan p =
        plan_bucket(ph.plan[j].K, ph.plan[j].A, ph.plan[j].B, 256, ph.plan[j].gram_space);
    if (p.keeps_xt) return;
    phase_add(q, p, ph.bucket[j]);
  }
  if (q.bytes <= kPhaseBytes) ph = q;
}

// Calls fn(phase) for each phase of the bucket list, in order (ns_mode: see
// ma_muon_hparams; Gram-space buckets form phases of their own).
template <class Fn>
ma_status for_each_phase(const ma_muon_bucket* buckets, int32_t n_buckets, int32_t ns_mode,
                         Fn&& fn) {
  Phase ph;
  for (int32_t i = 0; i < n_buckets; ++i) {
    if (buckets[i].K <= 0) continue;
    const BucketPlan p = plan_bucket(buckets[i].K, buckets[i].A, buckets[i].B, 0,
                                     wants_gram_space(ns_mode, buckets[i].A, buckets[i].B));
    if (ph.n > 0 && !phase_accepts(ph, p)) {
      promote(ph);
      const ma_status st = fn(ph);
      if (st != MA_OK) return st;
      ph = Phase();
    }
    phase_add(ph, p, i);
  }
  if (ph.n > 0) {
    promote(ph);
    return fn(ph);
  }
  return MA_OK;
}

// Tuned GEMM configurations ("DMuon: Efficient Distributed Muon Training with Near-Adam
// Overhead", section 2.4, autotuning per shape): one entry per phase shape (its buckets'
// K, padded sides, orientation and X^T choice), the configuration of the Gram,
// polynomial and combine launches (defaults: the library's rules).  Filled by
// ma_muon_tune / ma_muon_tune_configs, read by every Newton-Schulz run; process-wide,
// guarded by a mutex.
enum Product { kProdGram = 0, kProdPoly = 1, kProdCombine = 2 };
using Choices = std::array<GemmChoice, 3>;
std::mutex g_tune_mu;
std::map<std::vector<int64_t>, Choices> g_tune;

std::vector<int64_t> phase_key(const Phase& ph) {
  std::vector<int64_t> k{ph.n};
  for (int j = 0; j < ph.n; ++j) {
    const BucketPlan& p = ph.plan[j];
    k.insert(k.end(), {p.K, p.m_pad, p.n_pad, p.transposed ? 1 : 0, p.keeps_xt ? 1 : 0,
                       p.gram_space ? 1 : 0});
  }
  return k;
}

Choices tuned_choices(const Phase& ph) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  const auto it = g_tune.find(phase_key(ph));
  return it == g_tune.end() ? Choices{} : it->second;
}

// Tiles a product of this phase can run: 256 and 128 on a 256-padded phase (the
// combine of a phase that keeps X^T only its 256-tile configuration; 192-row combine
// tiles where every Gram side pads to a multiple of 192), 128 otherwise.
int tile_candidates(const Phase& ph, int prod, int (&out)[3]) {
  if (ph.tile != 256 || forced_tile()) {
    out[0] = ph.tile;
    return 1;
  }
  out[0] = 256;
  if (prod == kProdCombine && ph.plan[0].keeps_xt) return 1;
  out[1] = 128;
  if (prod != kProdCombine) return 2;
  for (int j = 0; j < ph.n; ++j)
    if (!combine_192_ok(ph.plan[j])) return 2;
  out[2] = 192;
  return 3;
}

bool tile_available(const Phase& ph, int prod, int tile) {
  int c[3];
  const int nc = tile_candidates(ph, prod, c);
  for (int i = 0; i < nc; ++i)
    if (c[i] == tile) return true;
  return false;
}

// Whether a product with this tile runs the 256-tile kernel whose pipeline can be chosen
// (the Gram-side products, and the combine of a phase that keeps X^T).
bool has_pipeline_choice(const Phase& ph, int prod, int tile) {
  if (forced_tile() ? forced_tile() != 256 : (tile ? tile : ph.tile) != 256 || ph.tile != 256)
    return false;
  return prod != kProdCombine || ph.plan[0].keeps_xt;
}

// A pinned configuration the phase can run: tile available (or 0), pipeline 0..2 (1, 2
// only where has_pipeline_choice), band 0..64, spread -1..1, xcd 0..3.
bool choice_valid(const Phase& ph, int prod, const GemmChoice& c) {
  if (c.tile != 0 && !tile_available(ph, prod, c.tile)) return false;
  if (c.pipeline < 0 || c.pipeline > 2) return false;
  if (c.pipeline != 0 && !has_pipeline_choice(ph, prod, c.tile)) return false;
  return c.band >= 0 && c.band <= 64 && c.spread >= -1 && c.spread <= 1 && c.xcd >= 0 &&
         c.xcd <= 3;
}

template <class T>
T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

// The GEMM operands of a phase's buckets for an iteration reading X[cur] (and writing
// X[cur ^ 1]).
void phase_groups(const Phase& ph, char* ws, int cur, NsGroup* g) {
  for (int j = 0; j < ph.n; ++j) {
    const BucketPlan& p = ph.plan[j];
    char* w = ws + ph.base[j];
    g[j].plan = &p;
    g[j].X = at<unsigned short>(w, p.off_x[cur]);
    g[j].Xn = at<unsigned short>(w, p.off_x[cur ^ 1]);
    g[j].XT = p.keeps_xt ? at<unsigned short>(w, p.off_xt[cur]) : nullptr;
    g[j].XTn = p.keeps_xt ? at<unsigned short>(w, p.off_xt[cur ^ 1]) : nullptr;
    g[j].R = at<unsigned short>(w, p.off_r);
    g[j].P = at<unsigned short>(w, p.off_p);
  }
}

// Newton-Schulz for every bucket of a phase whose unnormalised bf16 U sits in its X[0]
// (and, with no iteration, in its own orientation in X[1]) and whose normalisers
// inv[k] = 1 / (||U_k|| + eps) are in its workspace.  On
// return out[j] holds bucket j's result in the matrix's own orientation (row stride
// ldo[j]) and oscale[j] the per-matrix factor still to apply (inv when no iteration ran).
// The Gram-space form of the same iteration ("DMuon: Efficient Distributed Muon Training
// with Near-Adam Overhead", section 2.2, Gram Newton-Schulz), for a phase of buckets
// planned with gram_space and ns_steps >= 1.  With X_{k+1} = P_k X_k and P_k = a I +
// b R_k + c R_k^2 (R_k = X_k X_k^T), R_{k+1} = P_k R_k P_k and X_N = Q_N X_0 with
// Q_N = P_{N-1} ... P_0; every R_k, P_k, Q_k is a polynomial in R_0, so all of them and
// their products are symmetric and run on lower-triangle tiles.  Launches: the Gram of
// X_0 (normalised in its epilogue), per step the polynomial, Q <- P Q (from the second
// step), T = R P and R <- P T (all but the last step), then the combine X = inv Q U.
// Outputs as run_ns.
ma_status run_ns_gram_space(const Phase& ph, const ma_muon_hparams* hp, char* ws,
                            hipStream_t s, const unsigned short** out, int64_t* ldo,
                            const float** oscale) {
  // fp16 operands throughout ("DMuon", section 2.2, Gram-space recurrence): R carries
  // the squared spectrum, whose relative precision bf16's 8-bit significand loses on
  // wide Gram sides; fp16 keeps three more bits at the same MFMA rate, with powers of two
  // keeping every stored value in its normal range: X0 is stored as X0 * sx (by
  // prep_bucket), R and T = R P as R * rs, T * rs; P and Q unscaled (their eigenvalues lie
  // in [0.7, a] and [0, a^N] for the quintic on a normalised X0)
  NsGroup g[kMaxGemmGroups];
  SymProd sp[kMaxGemmGroups];
  const Choices tiles = tuned_choices(ph);
  phase_groups(ph, ws, 0, g);  // X = X_0 (fp16), Xn = the output, R = R_0
  auto buf = [&](int j, size_t off) { return at<unsigned short>(ws + ph.base[j], off); };
  // per-matrix factors written by the fp16 conversion (prep_bucket): the Gram's
  // 2^7 / sx_k (squared by its epilogue) and the last product's 1 / sx_k
  const float* gram_f[kMaxGemmGroups];
  const float* last_f[kMaxGemmGroups];
  for (int j = 0; j < ph.n; ++j) {
    const float* gsc = at<const float>(ws, ph.base[j] + ph.plan[j].off_gsc);
    gram_f[j] = gsc + ph.plan[j].K;
    last_f[j] = gsc + 2 * ph.plan[j].K;
  }
  const float rs = kGramSpaceRScale;
  hipError_t e = launch_gram(g, ph.n, gram_f, tiles[kProdGram], s, kTyF16);
  if (e != hipSuccess) return hip_fail(e, "gram launch");
  int rc = 0, qc = 0;  // current R (off_r / off_r2) and Q (off_q[qc])
  const int N = hp->ns_steps;
  for (int it = 0; it < N; ++it) {
    const NsCoeffs c = coeff_at(hp, it);
    // P_k; the first one is Q_1 itself (Q_0 = I), so it goes straight into Q[0]
    for (int j = 0; j < ph.n; ++j) {
      const BucketPlan& p = ph.plan[j];
      g[j].R = buf(j, rc ? p.off_r2 : p.off_r);
      g[j].P = buf(j, it == 0 ? p.off_q[0] : p.off_p);
    }
    // P = a I + b R + c R^2 from the stored rs R: b / rs and c / rs^2
    e = launch_poly(g, ph.n, c.a, c.b / rs, c.c / (rs * rs), tiles[kProdPoly], s, kTyF16);
    if (e != hipSuccess) return hip_fail(e, "poly launch");
    if (it > 0) {  // Q <- P Q
      for (int j = 0; j < ph.n; ++j)
        sp[j] = SymProd{&ph.plan[j], g[j].P, buf(j, ph.plan[j].off_q[qc]),
                        buf(j, ph.plan[j].off_q[qc ^ 1])};
      e = launch_sym(sp, ph.n, tiles[kProdPoly], s, kTyF16);
      if (e != hipSuccess) return hip_fail(e, "Q product launch");
      qc ^= 1;
    }
    if (it + 1 < N) {  // T = R P, then R <- P T (both carry the factor rs)
      for (int j = 0; j < ph.n; ++j)
        sp[j] = SymProd{&ph.plan[j], g[j].R, g[j].P, buf(j, ph.plan[j].off_t)};
      e = launch_sym(sp, ph.n, tiles[kProdPoly], s, kTyF16);
      if (e != hipSuccess) return hip_fail(e, "R P product launch");
      for (int j = 0; j < ph.n; ++j)
        sp[j] = SymProd{&ph.plan[j], g[j].P, buf(j, ph.plan[j].off_t),
                        buf(j, rc ? ph.plan[j].off_r : ph.plan[j].off_r2)};
      e = launch_sym(sp, ph.n, tiles[kProdPoly], s, kTyF16);
      if (e != hipSuccess) return hip_fail(e, "R update launch");
      rc ^= 1;
    }
  }
  // X_N = Q_N X_0 = Q_N (sx_k X0) / sx_k, in bf16 and in the parameter's orientation
  for (int j = 0; j < ph.n; ++j) g[j].P = buf(j, ph.plan[j].off_q[qc]);
  e = launch_combine(g, ph.n, last_f, true, tiles[kProdCombine], s, kTyF16ToBf16);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  for (int j = 0; j < ph.n; ++j) {
    const BucketPlan& p = ph.plan[j];
    out[j] = buf(j, (p.keeps_xt && p.transposed) ? p.off_xt[1] : p.off_x[1]);
    ldo[j] = p.transposed ? p.m_pad : p.n_pad;
    oscale[j] = nullptr;
  }
  return MA_OK;
}

ma_status run_ns(const Phase& ph, const ma_muon_hparams* hp, char* ws, hipStream_t s,
                 const unsigned short** out, int64_t* ldo, const float** oscale) {
  if (ph.plan[0].gram_space && hp->ns_steps > 0)
    return run_ns_gram_space(ph, hp, ws, s, out, ldo, oscale);
  NsGroup g[kMaxGemmGroups];
  const float* inv[kMaxGemmGroups];
  for (int j = 0; j < ph.n; ++j) inv[j] = at<const float>(ws, ph.base[j] + ph.plan[j].off_inv);
  const Choices tiles = tuned_choices(ph);
  int cur = 0;
  for (int it = 0; it < hp->ns_steps; ++it) {
    phase_groups(ph, ws, cur, g);
    const NsCoeffs c = coeff_at(hp, it);
    // the first iteration applies the normalisation X0 = inv U inside its products
    const float* const* sc = it == 0 ? inv : nullptr;
    hipError_t e = launch_gram(g, ph.n, sc, tiles[kProdGram], s);
    if (e != hipSuccess) return hip_fail(e, "gram launch");
    e = launch_poly(g, ph.n, c.a, c.b, c.c, tiles[kProdPoly], s);
    if (e != hipSuccess) return hip_fail(e, "poly launch");
    e = launch_combine(g, ph.n, sc, it + 1 == hp->ns_steps, tiles[kProdCombine], s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    cur ^= 1;
  }
  for (int j = 0; j < ph.n; ++j) {
    const BucketPlan& p = ph.plan[j];
    char* w = ws + ph.base[j];
    // own orientation: X (m_pad x n_pad) if not transposed, X^T (n_pad x m_pad) if it is;
    // written by the last combine, or by the cast when no iteration ran (one-orientation
    // buckets: the transposed bucket's own orientation then sits in X[1])
    if (p.keeps_xt) {
      out[j] = at<unsigned short>(w, p.transposed ? p.off_xt[cur] : p.off_x[cur]);
    } else {
      const int o = (hp->ns_steps == 0 && p.transposed) ? 1 : cur;
      out[j] = at<unsigned short>(w, p.off_x[o]);
    }
    ldo[j] = p.transposed ? p.m_pad : p.n_pad;
    oscale[j] = hp->ns_steps == 0 ? inv[j] : nullptr;
  }
  return MA_OK;
}

// momentum update + bf16 cast + norm of one bucket into its workspace region
ma_status prep_bucket(const BucketPlan& p, const float* grad, float* momentum,
                      const ma_muon_hparams* hp, char* w, hipStream_t s) {
  // X0 (the Gram-side orientation) in X[0], and X0^T in XT[0] for 256-tile buckets; a
  // one-orientation transposed bucket with no iteration also needs its own
  // orientation, in X[1]
  unsigned short* X0 = at<unsigned short>(w, p.off_x[0]);
  unsigned short* XT0 = p.keeps_xt ? at<unsigned short>(w, p.off_xt[0]) : nullptr;
  unsigned short* own = p.keeps_xt ? XT0
                        : (hp->ns_steps == 0 ? at<unsigned short>(w, p.off_x[1]) : nullptr);
  unsigned short* S = p.transposed ? own : X0;   // the matrix's own orientation
  unsigned short* T = p.transposed ? X0 : XT0;   // its transpose
  double* partials = at<double>(w, p.off_part);
  float* inv = at<float>(w, p.off_inv);
  int* shift = at<int>(w, p.off_shift);
  hipError_t e = launch_muon_prep(p, grad, momentum, momentum ? hp->momentum : 0.0f,
                                  momentum ? hp->nesterov : 0, partials, S, T, s);
  if (e != hipSuccess) return hip_fail(e, "momentum/cast launch");
  const bool f16 = p.gram_space && hp->ns_steps > 0;
  float* gsc = f16 ? at<float>(w, p.off_gsc) : nullptr;  // ||X0||, then the 2 K factors
  e = launch_norm_finalize(p, partials, hp->ns_eps, inv, shift, s, gsc);
  if (e != hipSuccess) return hip_fail(e, "norm launch");
  e = launch_rescale(p, S, T, shift, s);
  if (e != hipSuccess) return hip_fail(e, "rescale launch");
  if (f16) {
    // the Gram-space route iterates on fp16 operands: X0 = U / (||U|| + eps), times a
    // power of two that centres it in fp16's range, converted in place
    e = launch_to_f16(p, S, T, inv, gsc, p.gs_sx, gsc + p.K, s);
    if (e != hipSuccess) return hip_fail(e, "fp16 conversion launch");
  }
  return MA_OK;
}

// One phase of ma_muon_step: momentum, cast and norm of each bucket, the Newton-Schulz
// launches shared by the phase's buckets, then each bucket's update.
ma_status run_phase(const Phase& ph, const ma_muon_bucket* buckets, const ma_muon_hparams* hp,
                    char* ws, hipStream_t s) {
  for (int j = 0; j < ph.n; ++j) {
    const ma_muon_bucket& b = buckets[ph.bucket[j]];
    const ma_status st = prep_bucket(ph.plan[j], b.grad, b.momentum, hp, ws + ph.base[j], s);
    if (st != MA_OK) return st;
  }
  const unsigned short* O[kMaxGemmGroups];
  int64_t ldo[kMaxGemmGroups];
  const float* oscale[kMaxGemmGroups];
  const ma_status st = run_ns(ph, hp, ws, s, O, ldo, oscale);
  if (st != MA_OK) return st;
  for (int j = 0; j < ph.n; ++j) {
    const ma_muon_bucket& b = buckets[ph.bucket[j]];
    const double big = static_cast<double>(b.A > b.B ? b.A : b.B);
    const double scale =
        hp->scale_mode == 0
            ? 0.2 * std::sqrt(big)
            : std::sqrt(std::fmax(1.0, static_cast<double>(b.A) / static_cast<double>(b.B)));
    const hipError_t e = launch_muon_apply(ph.plan[j], b.param, O[j], oscale[j], ldo[j], hp->lr,
                                           hp->weight_decay, static_cast<float>(scale),
                                           hp->cautious_wd, s);
    if (e != hipSuccess) return hip_fail(e, "apply launch");
  }
  return MA_OK;
}

// ma_newton_schulz after its argument checks: cast, iterate, write out = NS(in) in fp32.
ma_status newton_schulz_body(const BucketPlan& p, const float* in, float* out,
                             const ma_muon_hparams* hp, char* ws, hipStream_t s) {
  Phase ph;
  phase_add(ph, p, 0);
  ma_status st = prep_bucket(p, in, nullptr, hp, ws, s);
  if (st != MA_OK) return st;
  const unsigned short* O[kMaxGemmGroups];
  int64_t ldo[kMaxGemmGroups];
  const float* oscale[kMaxGemmGroups];
  st = run_ns(ph, hp, ws, s, O, ldo, oscale);
  if (st != MA_OK) return st;
  const hipError_t e = launch_ns_extract(p, out, O[0], oscale[0], ldo[0], s);
  if (e != hipSuccess) return hip_fail(e, "extract launch");
  return MA_OK;
}

// The argument checks of ma_muon_step (everything but the workspace).
ma_status check_step_args(const ma_muon_bucket* buckets, int32_t n_buckets,
                          const ma_muon_hparams* hp) {
  ma_status st = check_hparams(hp);
  if (st != MA_OK) return st;
  if (n_buckets < 0) return fail(MA_ERR_INVALID_ARG, "n_buckets %d < 0", n_buckets);
  if (n_buckets > 0 && !buckets) return fail(MA_ERR_INVALID_ARG, "buckets is NULL");
  for (int32_t i = 0; i < n_buckets; ++i) {
    const ma_muon_bucket& b = buckets[i];
    st = check_shape(b.K, b.A, b.B);
    if (st != MA_OK) return fail(st, "bucket %d: %s", i, g_last_error.c_str());
    if (b.K == 0) continue;
    if (!b.param || !b.grad || !b.momentum)
      return fail(MA_ERR_INVALID_ARG, "bucket %d: NULL param, grad or momentum", i);
    if ((reinterpret_cast<uintptr_t>(b.param) | reinterpret_cast<uintptr_t>(b.grad) |
         reinterpret_cast<uintptr_t>(b.momentum)) & 3u)
      return fail(MA_ERR_INVALID_ARG, "bucket %d: pointers must be 4-byte aligned", i);
    const int64_t bytes = b.K * b.A * b.B * 4;
    const Range rp = range_of(b.param, bytes), rg = range_of(b.grad, bytes),
                rm = range_of(b.momentum, bytes);
    if (overlap(rp, rg) || overlap(rp, rm) || overlap(rg, rm))
      return fail(MA_ERR_INVALID_ARG, "bucket %d: param, grad and momentum overlap", i);
    // Across buckets: what one bucket writes (param, momentum) must not overlap
    // anything another bucket touches; gradients are read only and may alias.
    for (int32_t j = 0; j < i; ++j) {
      const ma_muon_bucket& o = buckets[j];
      if (o.K == 0) continue;
      const int64_t ob = o.K * o.A * o.B * 4;
      const Range op = range_of(o.param, ob), og = range_of(o.grad, ob),
                  om = range_of(o.momentum, ob);
      if (overlap(rp, op) || overlap(rp, og) || overlap(rp, om) || overlap(rm, op) ||
          overlap(rm, og) || overlap(rm, om) || overlap(rg, op) || overlap(rg, om))
        return fail(MA_ERR_INVALID_ARG, "buckets %d and %d overlap", j, i);
    }
  }
  return MA_OK;
}

// AdamW hyperparameter checks and the per-step constants of the kernels.
ma_status adamw_const(const ma_adamw_hparams* hp, AdamWConst* c) {
  if (!hp) return fail(MA_ERR_INVALID_ARG, "hparams is NULL");
  if (hp->step < 1) return fail(MA_ERR_INVALID_ARG, "step %lld < 1", (long long)hp->step);
  if (!finite(hp->lr) || !finite(hp->beta1) || !finite(hp->beta2) || !finite(hp->eps) ||
      !finite(hp->weight_decay))
    return fail(MA_ERR_INVALID_ARG, "non-finite AdamW hyperparameter");
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return fail(MA_ERR_INVALID_ARG, "betas must lie in [0, 1)");
  c->lr = hp->lr;
  c->beta1 = hp->beta1;
  c->beta2 = hp->beta2;
  c->one_m_beta1 = static_cast<float>(1.0 - static_cast<double>(hp->beta1));
  c->one_m_beta2 = static_cast<float>(1.0 - static_cast<double>(hp->beta2));
  c->eps = hp->eps;
  c->wd = hp->weight_decay;
  const double t = static_cast<double>(hp->step);
  c->inv_bc1 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(hp->beta1), t)));
  c->inv_bc2 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(hp->beta2), t)));
  c->decoupled = hp->decoupled ? 1 : 0;
  c->cautious = hp->cautious_wd ? 1 : 0;
  return MA_OK;
}

// Each device's copy of the static workspace (resolved once per device).
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ws[kMaxDevices] = {};

// Grid size limit of one launch (blocks), with the room the block-count arithmetic needs.
constexpr int64_t kMaxGridBlocks = (int64_t(1) << 31) - 4096;

// ---------------------------------------------------------------------------
// Plan check: replays the launches of a step with a recorder installed and checks, block
// by block, that every read and write stays inside the buffer it addresses, and that
// the GEMM blocks of each launch cover every output tile exactly once.
// ---------------------------------------------------------------------------
struct Region {
  uintptr_t lo, hi;
  std::string name;
};

class PlanChecker final : public LaunchRecorder {
 public:
  std::vector<Region> regions;
  std::string error;
  int64_t launches = 0, gemm_blocks = 0, tiles = 0;

  // the buffers of one phase (workspace regions of each bucket, and the caller's tensors)
  void set_phase(const Phase& ph, uintptr_t ws, size_t ws_bytes, const ma_muon_bucket* buckets,
                 bool has_momentum) {
    regions.clear();
    for (int j = 0; j < ph.n; ++j) {
      const BucketPlan& p = ph.plan[j];
      const uintptr_t b = ws + ph.base[j];
      const size_t xb = static_cast<size_t>(p.K * p.m_pad * p.n_pad) * 2;
      const size_t rb = static_cast<size_t>(p.K * p.m_pad * p.m_pad) * 2;
      const std::string t = "bucket " + std::to_string(ph.bucket[j]) + " ";
      add(b + p.off_x[0], xb, t + "X[0]");
      add(b + p.off_x[1], xb, t + "X[1]");
      if (p.keeps_xt) {
        add(b + p.off_xt[0], xb, t + "XT[0]");
        add(b + p.off_xt[1], xb, t + "XT[1]");
      }
      add(b + p.off_r, rb, t + "R");
      add(b + p.off_p, rb, t + "P");
      if (p.gram_space) {
        add(b + p.off_r2, rb, t + "R2");
        add(b + p.off_q[0], rb, t + "Q[0]");
        add(b + p.off_q[1], rb, t + "Q[1]");
        add(b + p.off_t, rb, t + "T");
        add(b + p.off_gsc, static_cast<size_t>(p.K) * 3 * 4, t + "Gram-space norms and factors");
      }
      add(b + p.off_part, static_cast<size_t>(p.K * p.nblk) * 8, t + "partials");
      add(b + p.off_inv, static_cast<size_t>(p.K) * 4, t + "inv");
      add(b + p.off_shift, static_cast<size_t>(p.K) * 4, t + "shift");
      const ma_muon_bucket& u = buckets[ph.bucket[j]];
      const size_t eb = static_cast<size_t>(u.K * u.A * u.B) * 4;
      add(reinterpret_cast<uintptr_t>(u.param), eb, t + "param");
      add(reinterpret_cast<uintptr_t>(u.grad), eb, t + "grad");
      if (has_momentum) add(reinterpret_cast<uintptr_t>(u.momentum), eb, t + "momentum");
      if (ph.base[j] + p.bytes > ws_bytes) fail_("bucket workspace beyond the workspace");
    }
    for (size_t i = 0; i < regions.size(); ++i)
      for (size_t k = i + 1; k < regions.size(); ++k)
        if (regions[i].lo < regions[k].hi && regions[k].lo < regions[i].hi)
          fail_("buffers " + regions[i].name + " and " + regions[k].name + " overlap");
  }

  void gemm(int epi, const TileShape& sh, const GemmTable& t) override {
    ++launches;
    const bool bt = epi == kCombine && sh.combine_reads_x;
    const int grid = t.start[t.ngroups];
    std::vector<std::vector<int>> seen(t.ngroups);
    for (int gi = 0; gi < t.ngroups; ++gi) {
      const GemmArgs& a = t.g[gi];
      if (a.kdim % sh.bk != 0) return fail_("contraction not a multiple of the stage depth");
      if (a.tiles_per_batch != (epi == kCombine ? a.tiles_m * a.tiles_n
                                                : a.tiles_m * (a.tiles_m + 1) / 2))
        return fail_("tile count does not match the tile grid");
      if (t.start[gi + 1] - t.start[gi] < a.tiles_per_batch * a.tiles_k || t.start[gi] % 8)
        return fail_("group block range too small or not on a multiple of 8");
      seen[gi].assign(static_cast<size_t>(a.tiles_per_batch) * a.tiles_k, 0);
    }
    for (int bid = 0; bid < grid && error.empty(); ++bid) {
      int gi, ti, tj;
      int64_t batch;
      if (!gemm_block_tile(t, epi, bid, gi, batch, ti, tj)) continue;
      ++gemm_blocks;
      const GemmArgs& a = t.g[gi];
      if (batch < 0 || batch >= a.tiles_k || ti < 0 || ti >= a.tiles_m || tj < 0 ||
          tj >= a.tiles_n || (epi != kCombine && tj > ti))
        return fail_("block " + std::to_string(bid) + " maps outside the tile grid");
      const int64_t slot = epi == kCombine ? static_cast<int64_t>(ti) * a.tiles_n + tj
                                           : static_cast<int64_t>(ti) * (ti + 1) / 2 + tj;
      if (++seen[gi][batch * a.tiles_per_batch + slot] != 1)
        return fail_("tile computed twice in one launch");
      const int64_t m0 = static_cast<int64_t>(ti) * sh.bm, n0 = static_cast<int64_t>(tj) * sh.bn;
      // operand panels
      win(a.A, batch * a.strideA + m0 * a.lda, (sh.bm - 1) * a.lda + a.kdim, "A operand");
      if (bt)
        win(a.B, batch * a.strideB + n0, (a.kdim - 1) * a.ldb + sh.bn, "B operand (X rows)");
      else
        win(a.B, batch * a.strideB + n0 * a.ldb, (sh.bn - 1) * a.ldb + a.kdim, "B operand");
      if (epi == kPoly)
        win(a.aux, batch * a.strideAux + n0 * a.ldaux + m0, (sh.bn - 1) * a.ldaux + sh.bm,
            "polynomial's R term");
      if (a.scale) winb(reinterpret_cast<uintptr_t>(a.scale + batch), 4, "scale");
      // results: the tile, and its transposed / mirrored copy
      const bool need_c = epi != kCombine || a.C;
      const bool need_t = epi == kCombine ? a.C2 != nullptr : ti != tj;
      if (need_c) win(a.C, batch * a.strideC + m0 * a.ldc + n0, (sh.bm - 1) * a.ldc + sh.bn, "C");
      if (need_t)
        win(a.C2, batch * a.strideC2 + n0 * a.ldc2 + m0, (sh.bn - 1) * a.ldc2 + sh.bm, "C2");
    }
    if (!error.empty()) return;
    for (int gi = 0; gi < t.ngroups; ++gi)
      for (int v : seen[gi])
        if (v != 1) return fail_("an output tile is not computed");
    for (int gi = 0; gi < t.ngroups; ++gi) tiles += static_cast<int64_t>(seen[gi].size());
  }

  void prep(const BucketPlan& p, const float* G, const float* M, const double* partials,
            const unsigned short* S, const unsigned short* T) override {
    ++launches;
    const int64_t Ap = p.transposed ? p.n_pad : p.m_pad, Bp = p.transposed ? p.m_pad : p.n_pad;
    if (Ap % kCastTile || Bp % kCastTile || (Ap / kCastTile) * (Bp / kCastTile) != p.nblk)
      return fail_("cast grid does not match the partial sums");
    winb(reinterpret_cast<uintptr_t>(G), p.K * p.A * p.B * 4, "gradient");
    if (M) winb(reinterpret_cast<uintptr_t>(M), p.K * p.A * p.B * 4, "momentum");
    winb(reinterpret_cast<uintptr_t>(partials), p.K * p.nblk * 8, "partials");
    if (S) win(S, 0, p.K * Ap * Bp, "cast S");
    if (T) win(T, 0, p.K * Ap * Bp, "cast T");
  }
  void norm(const BucketPlan& p, const double* partials, const float* inv,
            const int* shift, const float* x0norm) override {
    ++launches;
    winb(reinterpret_cast<uintptr_t>(partials), p.K * p.nblk * 8, "partials");
    winb(reinterpret_cast<uintptr_t>(inv), p.K * 4, "inv");
    winb(reinterpret_cast<uintptr_t>(shift), p.K * 4, "shift");
    if (x0norm) winb(reinterpret_cast<uintptr_t>(x0norm), p.K * 4, "x0norm");
  }
  void rescale(const BucketPlan& p, const unsigned short* S, const unsigned short* T,
               const int* shift) override {
    ++launches;
    if (S) win(S, 0, p.K * p.m_pad * p.n_pad, "rescaled S");
    if (T) win(T, 0, p.K * p.m_pad * p.n_pad, "rescaled T");
    winb(reinterpret_cast<uintptr_t>(shift), p.K * 4, "shift");
  }
  void to_f16(const BucketPlan& p, const unsigned short* S, const unsigned short* T,
              const float* inv, const float* x0norm, const float* gsc) override {
    ++launches;
    if (!p.gram_space) fail_("fp16 conversion of a bucket outside the Gram-space route");
    if (S) win(S, 0, p.K * p.m_pad * p.n_pad, "fp16 S");
    if (T) win(T, 0, p.K * p.m_pad * p.n_pad, "fp16 T");
    winb(reinterpret_cast<uintptr_t>(inv), p.K * 4, "inv");
    winb(reinterpret_cast<uintptr_t>(x0norm), p.K * 4, "x0norm");
    winb(reinterpret_cast<uintptr_t>(gsc), p.K * 2 * 4, "Gram-space factors");
  }
  void apply(const BucketPlan& p, const float* out, const unsigned short* O, const float* oscale,
             int64_t ldo) override {
    ++launches;
    if (ldo < p.B || (p.A - 1) * ldo + p.B > p.m_pad * p.n_pad)
      return fail_("orthogonalised matrix rows do not fit its slab");
    win(O, 0, (p.K - 1) * p.m_pad * p.n_pad + (p.A - 1) * ldo + p.B, "orthogonalised matrix");
    winb(reinterpret_cast<uintptr_t>(out), p.K * p.A * p.B * 4, "parameter / output");
    if (oscale) winb(reinterpret_cast<uintptr_t>(oscale), p.K * 4, "oscale");
  }

 private:
  void add(uintptr_t lo, size_t bytes, std::string name) {
    regions.push_back(Region{lo, lo + bytes, std::move(name)});
  }
  void fail_(const std::string& what) {
    if (error.empty()) error = what;
  }
  // `count` bf16 elements at element offset `off` from q
  void win(const unsigned short* q, int64_t off, int64_t count, const char* what) {
    if (!q) return fail_(std::string(what) + ": null pointer");
    if (off < 0 || count < 0) return fail_(std::string(what) + ": negative extent");
    winb(reinterpret_cast<uintptr_t>(q) + static_cast<uintptr_t>(off) * 2,
         static_cast<int64_t>(count) * 2, what);
  }
  void winb(uintptr_t lo, int64_t bytes, const char* what) {
    if (!error.empty()) return;
    for (const Region& r : regions)
      if (lo >= r.lo && lo < r.hi) {
        if (lo + static_cast<uintptr_t>(bytes) > r.hi)
          fail_(std::string(what) + " runs past the end of " + r.name);
        return;
      }
    fail_(std::string(what) + " starts outside every buffer");
  }
};

GemmChoice to_choice(const ma_gemm_config& c) {
  GemmChoice g;
  g.tile = c.tile;
  g.band = c.band;
  g.spread = c.spread;
  g.pipeline = c.pipeline;
  g.xcd = c.xcd;
  return g;
}

ma_gemm_config to_config(const GemmChoice& g) {
  return ma_gemm_config{g.tile, g.band, g.spread, g.pipeline, g.xcd};
}

// ma_muon_tune and ma_muon_tune_configs.  cfg: 3 entries per phase, input when reps = 0
// (pin), output when reps > 0 (search).  The search, per product of each phase, times
// candidates one dimension at a time from the defaults: the tile, then (for the 256-tile
// kernels with a choice) the pipeline, then the L2 band width (2, 4, 8 row panels), then
// (256- and 192-tiles) the DMA spreading, then the XCD block order; each candidate runs
// once to warm up and `reps`
// times between two HIP events on the phase's workspace operands (the buckets'
// gradients cast there first when every bucket of the phase gives one), and replaces the
// kept one only when at least 3 % faster.  tiles_only: the tile alone.
ma_status tune_impl(const ma_muon_bucket* buckets, int32_t n_buckets, const ma_muon_hparams* hp,
                    void* workspace, size_t workspace_bytes, void* stream, int32_t reps,
                    ma_gemm_config* cfg, bool tiles_only) {
  if (hp) {
    const ma_status st = check_hparams(hp);
    if (st != MA_OK) return st;
  }
  if (n_buckets < 0) return fail(MA_ERR_INVALID_ARG, "n_buckets %d < 0", n_buckets);
  if (n_buckets > 0 && !buckets) return fail(MA_ERR_INVALID_ARG, "buckets is NULL");
  if (reps < 0 || reps > 1000) return fail(MA_ERR_INVALID_ARG, "reps %d outside [0, 1000]", reps);
  for (int32_t i = 0; i < n_buckets; ++i) {
    const ma_status st = check_shape(buckets[i].K, buckets[i].A, buckets[i].B);
    if (st != MA_OK) return fail(st, "bucket %d: %s", i, g_last_error.c_str());
  }
  const int32_t mode = gs_mode(hp);
  if (reps == 0) {
    // pin: check every requested configuration first, then store (all default: forget)
    int phase = 0;
    ma_status st = for_each_phase(buckets, n_buckets, mode, [&](const Phase& ph) -> ma_status {
      for (int q = 0; q < 3; ++q)
        if (!choice_valid(ph, q, to_choice(cfg[3 * phase + q])))
          return fail(MA_ERR_INVALID_ARG,
                      "phase %d, product %d: configuration (tile %d, band %d, spread %d, "
                      "pipeline %d, xcd %d) is not available", phase, q, cfg[3 * phase + q].tile,
                      cfg[3 * phase + q].band, cfg[3 * phase + q].spread,
                      cfg[3 * phase + q].pipeline, cfg[3 * phase + q].xcd);
      ++phase;
      return MA_OK;
    });
    if (st != MA_OK) return st;
    phase = 0;
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return for_each_phase(buckets, n_buckets, mode, [&](const Phase& ph) -> ma_status {
      const Choices c{to_choice(cfg[3 * phase]), to_choice(cfg[3 * phase + 1]),
                      to_choice(cfg[3 * phase + 2])};
      if (c[0].is_default() && c[1].is_default() && c[2].is_default())
        g_tune.erase(phase_key(ph));
      else
        g_tune[phase_key(ph)] = c;
      ++phase;
      return MA_OK;
    });
  }
  const size_t need = ma_muon_workspace_bytes(buckets, n_buckets, hp);
  if (need > 0) {
    if (!workspace) return fail(MA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(MA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  int phases = 0;
  for_each_phase(buckets, n_buckets, mode, [&](const Phase&) { ++phases; return MA_OK; });
  if (phases == 0) return MA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const NsCoeffs c = hp ? coeff_at(hp, 0) : kQuintic;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t he = hipEventCreate(&e0);
  if (he == hipSuccess) he = hipEventCreate(&e1);
  if (he != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return hip_fail(he, "event create");
  }
  int phase = 0;
  const ma_status st = for_each_phase(buckets, n_buckets, mode, [&](const Phase& ph) -> ma_status {
    // the phase's operands: its gradients cast as ma_muon_step casts them, when given
    // (the matrix cores' power, and so the clock and the timing, depends on the data)
    bool have_grads = true;
    for (int j = 0; j < ph.n; ++j) have_grads = have_grads && buckets[ph.bucket[j]].grad;
    if (have_grads) {
      ma_muon_hparams cast_hp{};
      cast_hp.ns_eps = hp ? hp->ns_eps : 1e-7f;
      for (int j = 0; j < ph.n; ++j) {
        const ma_status s2 = prep_bucket(ph.plan[j], buckets[ph.bucket[j]].grad, nullptr,
                                         &cast_hp, ws + ph.base[j], s);
        if (s2 != MA_OK) return s2;
      }
    }
    NsGroup g[kMaxGemmGroups];
    phase_groups(ph, ws, 0, g);
    auto launch = [&](int q, const GemmChoice& ch) {
      switch (q) {
        case kProdGram: return launch_gram(g, ph.n, nullptr, ch, s);
        case kProdPoly: return launch_poly(g, ph.n, c.a, c.b, c.c, ch, s);
        default: return launch_combine(g, ph.n, nullptr, false, ch, s);
      }
    };
    // milliseconds of `reps` launches of one candidate (after one warm-up launch)
    auto time_of = [&](int q, const GemmChoice& ch, float* ms) -> hipError_t {
      hipError_t e = launch(q, ch);
      if (e == hipSuccess) e = hipEventRecord(e0, s);
      for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch(q, ch);
      if (e == hipSuccess) e = hipEventRecord(e1, s);
      if (e == hipSuccess) e = hipEventSynchronize(e1);
      if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
      return e;
    };
    Choices best{};
    for (int q = 0; q < 3; ++q) {
      GemmChoice cur{};
      float cur_ms = 0.0f;
      bool first = true;
      // a candidate replaces the one kept only when it is clearly faster: differences
      // of a few percent between launches of one configuration are noise
      constexpr float kMargin = 0.97f;
      auto consider = [&](const GemmChoice& cand) -> hipError_t {
        float ms = 0.0f;
        const hipError_t e = time_of(q, cand, &ms);
        if (e != hipSuccess) return e;
        if (first || ms < kMargin * cur_ms) {
          cur = cand;
          cur_ms = ms;
          first = false;
        }
        return hipSuccess;
      };
      // 1. tile
      int cand[3];
      const int nc = tile_candidates(ph, q, cand);
      for (int i = 0; i < nc; ++i) {
        GemmChoice t{};
        t.tile = cand[i];
        const hipError_t e = consider(t);
        if (e != hipSuccess) return hip_fail(e, "tuning launch");
      }
      if (!tiles_only) {
        // 2. pipeline of the 256-tile kernels
        const GemmChoice base = cur;
        if (has_pipeline_choice(ph, q, base.tile))
          for (int pl : {1, 2}) {
            GemmChoice t = base;
            t.pipeline = pl;
            const hipError_t e = consider(t);
            if (e != hipSuccess) return hip_fail(e, "tuning launch");
          }
        // 3. L2 band width of the tile order
        const GemmChoice base2 = cur;
        for (int band : {2, 4, 8}) {
          GemmChoice t = base2;
          t.band = band;
          const hipError_t e = consider(t);
          if (e != hipSuccess) return hip_fail(e, "tuning launch");
        }
        // 4. DMA spreading (256- and 192-tiles)
        const GemmChoice base3 = cur;
        const int tl = base3.tile ? base3.tile : ph.tile;
        if (tl >= 192 && !forced_tile())
          for (int sp : {0, 1}) {
            GemmChoice t = base3;
            t.spread = sp;
            const hipError_t e = consider(t);
            if (e != hipSuccess) return hip_fail(e, "tuning launch");
          }
        // 5. block order across the XCDs
        const GemmChoice base4 = cur;
        for (int x : {1, 2, 3}) {
          GemmChoice t = base4;
          t.xcd = x;
          const hipError_t e = consider(t);
          if (e != hipSuccess) return hip_fail(e, "tuning launch");
        }
      }
      best[q] = cur;
      cfg[3 * phase + q] = to_config(cur);
    }
    {
      std::lock_guard<std::mutex> lock(g_tune_mu);
      g_tune[phase_key(ph)] = best;
    }
    ++phase;
    return MA_OK;
  });
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

}  // namespace

LaunchRecorder*& launch_recorder() {
  static thread_local LaunchRecorder* r = nullptr;
  return r;
}

int forced_tile() {
  static const int t = [] {
    const char* env = std::getenv("MA_NS_TILE");
    const int v = env ? std::atoi(env) : 0;
    return (v == 128 || v == 256) ? v : 0;
  }();
  return t;
}

bool wants_gram_space(int32_t ns_mode, int64_t A, int64_t B) {
  // buckets whose long side is at least 3.5x the Gram side, in either orientation: there
  // the route does at most 27.5 m^3 of symmetric-count work per matrix against the
  // printed iteration's 57.5 m^3 (five steps), and its fp16 error stayed within 1.3e-2
  // of the exact iteration on conditioned gradients over many seeds (2-7e-3 at the
  // workloads' sizes); at 3:1 conditioned gradients reached 2.0-2.5e-2 on Gram sides of
  // 64 to 256, so squarer buckets run the printed iteration
  const int64_t m = A < B ? A : B, n = A < B ? B : A;
  return ns_mode == 1 && kGramSpaceAspectDen * n >= kGramSpaceAspectNum * m;
}

// Whether every value the fp16 Gram-space route stores stays inside fp16's range for
// these coefficients and steps.  X0 is normalised, so the iterate's singular values start
// in [0, 1]; each step maps sigma to p(sigma) = sigma q(sigma^2), q(t) = a + b t + c t^2,
// so their bound s becomes max |p| over [0, s].  R (eigenvalues sigma^2 <= s^2) and R P
// (sigma p(sigma)) are stored times kGramSpaceRScale; P (q) and Q (the product of the
// steps' q) unscaled, Q bounded by the product of max |q| over [0, s^2] (reached on a
// zero singular value, where Q grows as a^N).  Symmetric entries are bounded by the
// largest eigenvalue modulus; sampled on a grid, with a margin of 2 below fp16's maximum.
bool gram_space_range_ok(const ma_muon_hparams* hp) {
  constexpr int kGrid = 4096;
  constexpr double kLimit = 32768.0;
  const double rs = kGramSpaceRScale;
  if (hp->ns_steps < 0 || hp->ns_steps > MA_MAX_NS_STEPS) return false;
  double s = 1.0, q_prod = 1.0;
  for (int it = 0; it < hp->ns_steps; ++it) {
    const NsCoeffs c = coeff_at(hp, it);
    double pmax = 0.0, qmax = 0.0;
    for (int i = 0; i <= kGrid; ++i) {
      const double sig = s * i / kGrid, t = sig * sig;
      const double q = c.a + c.b * t + c.c * t * t;
      qmax = std::max(qmax, std::fabs(q));
      pmax = std::max(pmax, std::fabs(sig * q));
    }
    q_prod *= qmax;
    // (written so that a NaN coefficient fails the test too)
    if (!(s * s * rs <= kLimit && s * pmax * rs <= kLimit && q_prod <= kLimit)) return false;
    s = pmax;
  }
  return true;
}

int32_t gs_mode(const ma_muon_hparams* hp) {
  return (hp && hp->ns_mode == 1 && gram_space_range_ok(hp)) ? 1 : 0;
}

float gram_space_sx(int64_t m, int64_t n) {
  int e = 0;
  while (e < 14 && (int64_t{1} << (2 * (e + 1))) <= m * n) ++e;
  return static_cast<float>(int64_t{1} << e);
}

BucketPlan plan_bucket(int64_t K, int64_t A, int64_t B, int tile, bool gram_space) {
  BucketPlan p{};
  p.K = K;
  p.A = A;
  p.B = B;
  p.transposed = A > B;
  p.m = p.transposed ? B : A;
  p.n = p.transposed ? A : B;
  p.tile = tile ? tile : pick_tile(K, p.m, p.n);
  if (const int t = forced_tile()) p.tile = t;
  p.m_pad = round_up(p.m, p.tile);
  p.n_pad = round_up(p.n, p.tile);
  p.nblk = (p.m_pad / kCastTile) * (p.n_pad / kCastTile);
  const size_t xb = static_cast<size_t>(K * p.m_pad * p.n_pad) * 2;
  const size_t rb = static_cast<size_t>(K * p.m_pad * p.m_pad) * 2;
  size_t off = 0;
  p.keeps_xt = p.tile == 256 && p.m_pad > 2048;
  for (int i = 0; i < 2; ++i) {
    p.off_x[i] = off;
    off = align256(off + xb);
    p.off_xt[i] = off;
    if (p.keeps_xt) off = align256(off + xb);
  }
  p.off_r = off;
  off = align256(off + rb);
  p.off_p = off;
  off = align256(off + rb);
  p.gram_space = gram_space;
  p.gs_sx = gram_space ? gram_space_sx(p.m, p.n) : 1.0f;
  p.off_r2 = p.off_q[0] = p.off_q[1] = p.off_t = p.off_gsc = 0;
  if (gram_space) {
    p.off_r2 = off;
    off = align256(off + rb);
    for (int i = 0; i < 2; ++i) {
      p.off_q[i] = off;
      off = align256(off + rb);
    }
    p.off_t = off;
    off = align256(off + rb);
    p.off_gsc = off;
    off = align256(off + static_cast<size_t>(K) * 3 * 4);
  }
  p.off_part = off;
  off = align256(off + static_cast<size_t>(K * p.nblk) * 8);
  p.off_inv = off;
  off = align256(off + static_cast<size_t>(K) * 4);
  p.off_shift = off;
  off = align256(off + static_cast<size_t>(K) * 4);
  p.bytes = off;
  return p;
}

}  // namespace ma

using namespace ma;

extern "C" {

int ma_abi_version(void) { return MA_ABI_VERSION; }

const char* ma_status_string(int status) {
  switch (status) {
    case MA_OK: return "ok";
    case MA_ERR_INVALID_ARG: return "invalid argument";
    case MA_ERR_UNSUPPORTED: return "unsupported";
    case MA_ERR_WORKSPACE: return "workspace missing or too small";
    case MA_ERR_HIP: return "HIP error";
    case MA_ERR_INTERNAL: return "internal check failed";
    default: return "unknown status";
  }
}

const char* ma_last_error(void) { return g_last_error.c_str(); }

ma_status ma_muon_route_of(int64_t A, int64_t B, const ma_muon_hparams* hp, ma_muon_route* out) {
  g_last_error.clear();
  if (!out) return fail(MA_ERR_INVALID_ARG, "out is NULL");
  if (A < 1 || B < 1) return fail(MA_ERR_INVALID_ARG, "matrix shape %lld x %lld", (long long)A, (long long)B);
  const int steps = hp ? hp->ns_steps : 5;
  if (steps < 0 || steps > MA_MAX_NS_STEPS) return fail(MA_ERR_INVALID_ARG, "ns_steps %d", steps);
  *out = route_of(plan_bucket(1, A, B, 0, wants_gram_space(gs_mode(hp), A, B)), steps);
  return MA_OK;
}

size_t ma_muon_workspace_bytes(const ma_muon_bucket* buckets, int32_t n_buckets,
                               const ma_muon_hparams* hp) {
  if (n_buckets <= 0 || !buckets) return 0;
  for (int32_t i = 0; i < n_buckets; ++i)
    if (buckets[i].K > 0 && (buckets[i].A < 1 || buckets[i].B < 1)) return 0;
  size_t need = 0;
  for_each_phase(buckets, n_buckets, gs_mode(hp), [&](const Phase& ph) {
    if (ph.bytes > need) need = ph.bytes;
    return MA_OK;
  });
  return need;
}

int32_t ma_muon_phases(const ma_muon_bucket* buckets, int32_t n_buckets,
                       const ma_muon_hparams* hp, int32_t* phase_of) {
  g_last_error.clear();
  if (n_buckets < 0) return fail(MA_ERR_INVALID_ARG, "n_buckets %d < 0", n_buckets);
  if (n_buckets > 0 && !buckets) return fail(MA_ERR_INVALID_ARG, "buckets is NULL");
  for (int32_t i = 0; i < n_buckets; ++i) {
    const ma_status st = check_shape(buckets[i].K, buckets[i].A, buckets[i].B);
    if (st != MA_OK) return fail(st, "bucket %d: %s", i, g_last_error.c_str());
    if (phase_of) phase_of[i] = -1;
  }
  int32_t count = 0;
  for_each_phase(buckets, n_buckets, gs_mode(hp), [&](const Phase& ph) {
    if (phase_of)
      for (int j = 0; j < ph.n; ++j) phase_of[ph.bucket[j]] = count;
    ++count;
    return MA_OK;
  });
  return count;
}

ma_status ma_muon_step(const ma_muon_bucket* buckets, int32_t n_buckets,
                       const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                       void* stream, ma_muon_route* route_out) {
  g_last_error.clear();
  const ma_status st = check_step_args(buckets, n_buckets, hp);
  if (st != MA_OK) return st;
  const size_t need = ma_muon_workspace_bytes(buckets, n_buckets, hp);
  if (need > 0) {
    if (!workspace) return fail(MA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(MA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  if (route_out) {
    // from the plans the phases run (a phase may re-plan its buckets' tile)
    for (int32_t i = 0; i < n_buckets; ++i) route_out[i] = ma_muon_route{0, 0, 0, 0, 0, 0, 0};
    for_each_phase(buckets, n_buckets, gs_mode(hp), [&](const Phase& ph) {
      for (int j = 0; j < ph.n; ++j) route_out[ph.bucket[j]] = route_of(ph.plan[j], hp->ns_steps);
      return MA_OK;
    });
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  return for_each_phase(buckets, n_buckets, gs_mode(hp), [&](const Phase& ph) {
    return run_phase(ph, buckets, hp, ws, s);
  });
}

size_t ma_newton_schulz_workspace_bytes(int64_t K, int64_t A, int64_t B) {
  if (K <= 0 || A < 1 || B < 1) return 0;
  // enough for either ns_mode (the Gram-space plan adds four m x m buffers)
  const size_t plain = plan_bucket(K, A, B).bytes;
  const size_t gs = plan_bucket(K, A, B, 0, wants_gram_space(1, A, B)).bytes;
  return plain > gs ? plain : gs;
}

ma_status ma_newton_schulz(const float* in, float* out, int64_t K, int64_t A, int64_t B,
                           const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_last_error.clear();
  ma_status st = check_hparams(hp);
  if (st != MA_OK) return st;
  st = check_shape(K, A, B);
  if (st != MA_OK) return st;
  if (K == 0) return MA_OK;
  if (!in || !out) return fail(MA_ERR_INVALID_ARG, "NULL in or out");
  if ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 3u)
    return fail(MA_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  const int64_t bytes = K * A * B * 4;
  if (overlap(range_of(in, bytes), range_of(out, bytes)))
    return fail(MA_ERR_INVALID_ARG, "in and out overlap");
  const BucketPlan p = plan_bucket(K, A, B, 0, wants_gram_space(gs_mode(hp), A, B));
  if (!workspace) return fail(MA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", p.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.bytes)
    return fail(MA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, p.bytes);
  return newton_schulz_body(p, in, out, hp, static_cast<char*>(workspace),
                            static_cast<hipStream_t>(stream));
}

ma_status ma_muon_tune(const ma_muon_bucket* buckets, int32_t n_buckets,
                       const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                       void* stream, int32_t reps, int32_t* tiles) {
  // the tile-only form of ma_muon_tune_configs
  g_last_error.clear();
  if (reps == 0 && !tiles) return fail(MA_ERR_INVALID_ARG, "tiles is NULL with reps 0");
  const int32_t nph = ma_muon_phases(buckets, n_buckets, hp, nullptr);
  if (nph < 0) return static_cast<ma_status>(nph);
  std::vector<ma_gemm_config> cfg(static_cast<size_t>(3 * std::max(nph, 1)),
                                  ma_gemm_config{0, 0, -1, 0, 0});
  if (reps == 0)
    for (int i = 0; i < 3 * nph; ++i) cfg[i].tile = tiles[i];
  const ma_status st = tune_impl(buckets, n_buckets, hp, workspace, workspace_bytes, stream, reps,
                                 cfg.data(), /*tiles_only=*/true);
  if (st == MA_OK && reps > 0 && tiles)
    for (int i = 0; i < 3 * nph; ++i) tiles[i] = cfg[i].tile;
  return st;
}

ma_status ma_muon_tune_configs(const ma_muon_bucket* buckets, int32_t n_buckets,
                               const ma_muon_hparams* hp, void* workspace,
                               size_t workspace_bytes, void* stream, int32_t reps,
                               ma_gemm_config* configs) {
  g_last_error.clear();
  if (reps == 0 && !configs) return fail(MA_ERR_INVALID_ARG, "configs is NULL with reps 0");
  const int32_t nph = ma_muon_phases(buckets, n_buckets, hp, nullptr);
  if (nph < 0) return static_cast<ma_status>(nph);
  std::vector<ma_gemm_config> cfg(static_cast<size_t>(3 * std::max(nph, 1)),
                                  ma_gemm_config{0, 0, -1, 0, 0});
  if (reps == 0)
    for (int i = 0; i < 3 * nph; ++i) cfg[i] = configs[i];
  const ma_status st = tune_impl(buckets, n_buckets, hp, workspace, workspace_bytes, stream, reps,
                                 cfg.data(), /*tiles_only=*/false);
  if (st == MA_OK && reps > 0 && configs)
    for (int i = 0; i < 3 * nph; ++i) configs[i] = cfg[i];
  return st;
}

void ma_muon_tune_reset(void) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  g_tune.clear();
}

ma_status ma_muon_static_init(void) {
  g_last_error.clear();
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_ws[dev]) return MA_OK;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
    return fail(MA_ERR_HIP, "static workspace address %p is null or not 256-byte aligned", ptr);
  g_static_ws[dev] = ptr;
  return MA_OK;
}

ma_status ma_muon_step_static(const ma_muon_bucket* buckets, int32_t n_buckets,
                              const ma_muon_hparams* hp, void* stream,
                              ma_muon_route* route_out) {
  g_last_error.clear();
  ma_status st = check_step_args(buckets, n_buckets, hp);
  if (st != MA_OK) return st;
  const size_t need = ma_muon_workspace_bytes(buckets, n_buckets, hp);
  if (need > MA_STATIC_WORKSPACE_BYTES)
    return fail(MA_ERR_WORKSPACE,
                "these buckets need %zu bytes of workspace, above the static workspace's %zu "
                "(use ma_muon_step with a caller workspace)",
                need, static_cast<size_t>(MA_STATIC_WORKSPACE_BYTES));
  st = ma_muon_static_init();
  if (st != MA_OK) return st;
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_static_mu);
    ws = g_static_ws[dev];
  }
  return ma_muon_step(buckets, n_buckets, hp, ws, MA_STATIC_WORKSPACE_BYTES, stream, route_out);
}

ma_status ma_muon_check_plan(const ma_muon_bucket* buckets, int32_t n_buckets,
                             const ma_muon_hparams* hp, int32_t what, ma_plan_report* out) {
  g_last_error.clear();
  if (what != 0 && what != 1) return fail(MA_ERR_INVALID_ARG, "what %d is not 0 or 1", what);
  if (n_buckets < 0) return fail(MA_ERR_INVALID_ARG, "n_buckets %d < 0", n_buckets);
  if (n_buckets > 0 && !buckets) return fail(MA_ERR_INVALID_ARG, "buckets is NULL");
  if (what == 1 && n_buckets < 1) return fail(MA_ERR_INVALID_ARG, "no bucket to orthogonalise");
  // synthetic, disjoint, 256-byte aligned tensors and workspace (never dereferenced)
  std::vector<ma_muon_bucket> bk(static_cast<size_t>(n_buckets));
  uintptr_t addr = uintptr_t(1) << 44;
  auto take = [&](int64_t bytes) {
    const uintptr_t a = addr;
    addr += (static_cast<uintptr_t>(bytes) + 511) & ~static_cast<uintptr_t>(255);
    return a;
  };
  for (int32_t i = 0; i < n_buckets; ++i) {
    bk[i] = ma_muon_bucket{buckets[i].K, buckets[i].A, buckets[i].B, nullptr, nullptr, nullptr};
    const ma_status st = check_shape(bk[i].K, bk[i].A, bk[i].B);
    if (st != MA_OK) return fail(st, "bucket %d: %s", i, g_last_error.c_str());
    if (bk[i].K == 0) continue;
    const int64_t bytes = bk[i].K * bk[i].A * bk[i].B * 4;
    bk[i].param = reinterpret_cast<float*>(take(bytes));
    bk[i].grad = reinterpret_cast<const float*>(take(bytes));
    bk[i].momentum = reinterpret_cast<float*>(take(bytes));
  }
  ma_status st = what == 0 ? check_step_args(bk.data(), n_buckets, hp) : check_hparams(hp);
  if (st != MA_OK) return st;
  PlanChecker chk;
  struct Install {
    explicit Install(LaunchRecorder* r) { launch_recorder() = r; }
    ~Install() { launch_recorder() = nullptr; }
  } install(&chk);
  const uintptr_t ws = take(0);
  if (what == 0) {
    const size_t need = ma_muon_workspace_bytes(bk.data(), n_buckets, hp);
    st = for_each_phase(bk.data(), n_buckets, gs_mode(hp), [&](const Phase& ph) -> ma_status {
      chk.set_phase(ph, ws, need, bk.data(), true);
      if (chk.error.empty()) {
        const ma_status s2 = run_phase(ph, bk.data(), hp, reinterpret_cast<char*>(ws), nullptr);
        if (s2 != MA_OK) return s2;
      }
      return chk.error.empty() ? MA_OK : MA_ERR_INTERNAL;
    });
  } else if (bk[0].K > 0) {
    const ma_muon_bucket& b = bk[0];
    const BucketPlan p = plan_bucket(b.K, b.A, b.B, 0, wants_gram_space(gs_mode(hp), b.A, b.B));
    Phase ph;
    phase_add(ph, p, 0);
    chk.set_phase(ph, ws, p.bytes, bk.data(), false);
    if (chk.error.empty()) {
      // in = the gradient, out = the parameter tensor
      st = newton_schulz_body(p, b.grad, b.param, hp, reinterpret_cast<char*>(ws), nullptr);
      if (st != MA_OK) return st;
    }
    if (!chk.error.empty()) st = MA_ERR_INTERNAL;
  }
  if (st == MA_ERR_INTERNAL || !chk.error.empty())
    return fail(MA_ERR_INTERNAL, "plan check: %s", chk.error.c_str());
  if (st != MA_OK) return st;
  if (out) *out = ma_plan_report{chk.launches, chk.gemm_blocks, chk.tiles};
  return MA_OK;
}

ma_status ma_muon_ns_time(const ma_muon_bucket* buckets, int32_t n_buckets,
                          const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                          void* stream, int32_t reps, float* phase_ms) {
  g_last_error.clear();
  ma_status st = check_hparams(hp);
  if (st != MA_OK) return st;
  if (n_buckets < 0) return fail(MA_ERR_INVALID_ARG, "n_buckets %d < 0", n_buckets);
  if (n_buckets > 0 && !buckets) return fail(MA_ERR_INVALID_ARG, "buckets is NULL");
  if (reps < 1 || reps > 1000) return fail(MA_ERR_INVALID_ARG, "reps %d outside [1, 1000]", reps);
  if (!phase_ms) return fail(MA_ERR_INVALID_ARG, "phase_ms is NULL");
  for (int32_t i = 0; i < n_buckets; ++i) {
    st = check_shape(buckets[i].K, buckets[i].A, buckets[i].B);
    if (st != MA_OK) return fail(st, "bucket %d: %s", i, g_last_error.c_str());
    if (buckets[i].K > 0 && (!buckets[i].grad || (reinterpret_cast<uintptr_t>(buckets[i].grad) & 3u)))
      return fail(MA_ERR_INVALID_ARG, "bucket %d: gradient NULL or not 4-byte aligned", i);
  }
  const size_t need = ma_muon_workspace_bytes(buckets, n_buckets, hp);
  if (need > 0) {
    if (!workspace) return fail(MA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(MA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t he = hipEventCreate(&e0);
  if (he == hipSuccess) he = hipEventCreate(&e1);
  if (he != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return hip_fail(he, "event create");
  }
  int phase = 0;
  st = for_each_phase(buckets, n_buckets, gs_mode(hp), [&](const Phase& ph) -> ma_status {
    double total = 0.0;
    for (int r = 0; r < reps; ++r) {
      for (int j = 0; j < ph.n; ++j) {
        const ma_status s2 = prep_bucket(ph.plan[j], buckets[ph.bucket[j]].grad, nullptr, hp,
                                         ws + ph.base[j], s);
        if (s2 != MA_OK) return s2;
      }
      const unsigned short* O[kMaxGemmGroups];
      int64_t ldo[kMaxGemmGroups];
      const float* oscale[kMaxGemmGroups];
      hipError_t e = hipEventRecord(e0, s);
      if (e != hipSuccess) return hip_fail(e, "event record");
      const ma_status s2 = run_ns(ph, hp, ws, s, O, ldo, oscale);
      if (s2 != MA_OK) return s2;
      e = hipEventRecord(e1, s);
      if (e == hipSuccess) e = hipEventSynchronize(e1);
      float ms = 0.0f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
      if (e != hipSuccess) return hip_fail(e, "timing");
      total += ms;
    }
    phase_ms[phase++] = static_cast<float>(total / reps);
    return MA_OK;
  });
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

ma_status ma_stream_probe(const float* const* in, int32_t reads, float* const* out,
                          int32_t writes, int64_t n, void* stream) {
  g_last_error.clear();
  if (reads < 1 || reads > 4 || writes < 0 || writes > 3)
    return fail(MA_ERR_INVALID_ARG, "reads %d / writes %d outside 1..4 / 0..3", reads, writes);
  if (n < 0 || n % 4) return fail(MA_ERR_INVALID_ARG, "n = %lld is not a multiple of 4", (long long)n);
  if (n == 0) return MA_OK;
  if (!in || (writes > 0 && !out)) return fail(MA_ERR_INVALID_ARG, "NULL pointer table");
  // an output may be exactly one of the inputs (streamed in place, as the AdamW step
  // updates p, m and v); any other overlap is rejected
  std::vector<Range> rs;
  for (int i = 0; i < reads + writes; ++i) {
    const void* q = i < reads ? static_cast<const void*>(in[i]) : static_cast<const void*>(out[i - reads]);
    if (!q || (reinterpret_cast<uintptr_t>(q) & 15u))
      return fail(MA_ERR_INVALID_ARG, "array %d NULL or not 16-byte aligned", i);
    const Range r = range_of(q, n * 4);
    for (size_t k = 0; k < rs.size(); ++k) {
      const bool in_place = i >= reads && static_cast<int>(k) < reads && rs[k].lo == r.lo;
      if (overlap(r, rs[k]) && !in_place) return fail(MA_ERR_INVALID_ARG, "arrays overlap");
    }
    rs.push_back(r);
  }
  const hipError_t e = launch_stream_probe(in, reads, out, writes, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return MA_OK;
}

ma_status ma_mfma_probe(const void* operands, int32_t blocks, int32_t iters, float* out,
                        uint64_t* clocks, void* stream) {
  g_last_error.clear();
  if (!operands || (reinterpret_cast<uintptr_t>(operands) & 15u))
    return fail(MA_ERR_INVALID_ARG, "operands NULL or not 16-byte aligned");
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u))
    return fail(MA_ERR_INVALID_ARG, "out NULL or not 4-byte aligned");
  if (clocks && (reinterpret_cast<uintptr_t>(clocks) & 7u))
    return fail(MA_ERR_INVALID_ARG, "clocks not 8-byte aligned");
  if (blocks < 1 || blocks > 65535) return fail(MA_ERR_INVALID_ARG, "blocks = %d outside 1..65535", blocks);
  if (iters < 1 || iters > (1 << 22)) return fail(MA_ERR_INVALID_ARG, "iters = %d outside 1..2^22", iters);
  const hipError_t e = launch_mfma_probe(operands, blocks, iters, out,
                                         reinterpret_cast<unsigned long long*>(clocks),
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return MA_OK;
}

ma_status ma_adamw_step(float* param, const float* grad, float* exp_avg, float* exp_avg_sq,
                        int64_t n, const ma_adamw_hparams* hp, void* stream) {
  g_last_error.clear();
  AdamWConst c;
  const ma_status st = adamw_const(hp, &c);
  if (st != MA_OK) return st;
  if (n < 0) return fail(MA_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (n == 0) return MA_OK;
  if (!param || !grad || !exp_avg || !exp_avg_sq)
    return fail(MA_ERR_INVALID_ARG, "NULL param, grad, exp_avg or exp_avg_sq");
  if ((reinterpret_cast<uintptr_t>(param) | reinterpret_cast<uintptr_t>(grad) |
       reinterpret_cast<uintptr_t>(exp_avg) | reinterpret_cast<uintptr_t>(exp_avg_sq)) & 3u)
    return fail(MA_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  const Range r[4] = {range_of(param, n * 4), range_of(grad, n * 4), range_of(exp_avg, n * 4),
                      range_of(exp_avg_sq, n * 4)};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(r[i], r[j])) return fail(MA_ERR_INVALID_ARG, "param/grad/exp_avg/exp_avg_sq overlap");
  const hipError_t e = launch_adamw(param, grad, exp_avg, exp_avg_sq, n, c,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "adamw launch");
  return MA_OK;
}

ma_status ma_adamw_step_multi(const ma_adamw_segment* segs, int32_t n_segs,
                              const ma_adamw_hparams* hp, void* stream) {
  g_last_error.clear();
  AdamWConst c;
  ma_status st = adamw_const(hp, &c);
  if (st != MA_OK) return st;
  if (n_segs < 0) return fail(MA_ERR_INVALID_ARG, "n_segs %d < 0", n_segs);
  if (n_segs > 0 && !segs) return fail(MA_ERR_INVALID_ARG, "segs is NULL");
  // every segment on its own, then no write range may overlap any other range (a sweep
  // over the ranges sorted by start: a range overlaps an earlier one iff it starts
  // before the largest end seen so far)
  struct Span {
    uintptr_t lo, hi;
    bool write;
  };
  std::vector<Span> spans;
  spans.reserve(static_cast<size_t>(n_segs) * 4);
  for (int32_t i = 0; i < n_segs; ++i) {
    const ma_adamw_segment& g = segs[i];
    if (g.n < 0) return fail(MA_ERR_INVALID_ARG, "segment %d: n = %lld < 0", i, (long long)g.n);
    if (g.n == 0) continue;
    if (!g.param || !g.grad || !g.exp_avg || !g.exp_avg_sq)
      return fail(MA_ERR_INVALID_ARG, "segment %d: NULL pointer", i);
    if ((reinterpret_cast<uintptr_t>(g.param) | reinterpret_cast<uintptr_t>(g.grad) |
         reinterpret_cast<uintptr_t>(g.exp_avg) | reinterpret_cast<uintptr_t>(g.exp_avg_sq)) & 3u)
      return fail(MA_ERR_INVALID_ARG, "segment %d: pointers must be 4-byte aligned", i);
    const int64_t b = g.n * 4;
    spans.push_back({range_of(g.param, b).lo, range_of(g.param, b).hi, true});
    spans.push_back({range_of(g.grad, b).lo, range_of(g.grad, b).hi, false});
    spans.push_back({range_of(g.exp_avg, b).lo, range_of(g.exp_avg, b).hi, true});
    spans.push_back({range_of(g.exp_avg_sq, b).lo, range_of(g.exp_avg_sq, b).hi, true});
  }
  std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  uintptr_t end_any = 0, end_write = 0;
  for (const Span& x : spans) {
    if (x.lo < (x.write ? end_any : end_write))
      return fail(MA_ERR_INVALID_ARG, "segments overlap (a written range meets another range)");
    end_any = std::max(end_any, x.hi);
    if (x.write) end_write = std::max(end_write, x.hi);
  }
  // launches of up to kMaxAdamWSegs segments, in order
  AdamWSegTable t{};
  t.c = c;
  auto flush = [&]() -> ma_status {
    if (t.nseg == 0) return MA_OK;
    const hipError_t e = launch_adamw_multi(t, static_cast<hipStream_t>(stream));
    t.nseg = 0;
    t.block_start[0] = 0;
    if (e != hipSuccess) return hip_fail(e, "adamw multi launch");
    return MA_OK;
  };
  for (int32_t i = 0; i < n_segs; ++i) {
    const ma_adamw_segment& g = segs[i];
    if (g.n == 0) continue;
    const int64_t nb = adamw_multi_blocks(g.n);
    if (t.nseg == kMaxAdamWSegs || t.block_start[t.nseg] + nb > kMaxGridBlocks) {
      st = flush();
      if (st != MA_OK) return st;
    }
    if (nb > kMaxGridBlocks)
      return fail(MA_ERR_UNSUPPORTED, "segment %d: %lld elements exceed one launch", i,
                  (long long)g.n);
    const int k = t.nseg;
    t.p[k] = g.param;
    t.g[k] = g.grad;
    t.m[k] = g.exp_avg;
    t.v[k] = g.exp_avg_sq;
    t.n[k] = g.n;
    t.vec[k] = ((reinterpret_cast<uintptr_t>(g.param) | reinterpret_cast<uintptr_t>(g.grad) |
                 reinterpret_cast<uintptr_t>(g.exp_avg) | reinterpret_cast<uintptr_t>(g.exp_avg_sq)) &
                15u) == 0;
    t.block_start[k + 1] = t.block_start[k] + nb;
    t.nseg = k + 1;
  }
  return flush();
}

}  // extern "C"
