/*
 * muon_adamw.h -- C ABI of the hybrid Muon + AdamW optimizer step on MI355X (gfx950).
 *
 * The library (libmuonadamw.so) performs one optimizer step:
 *
 *   ma_muon_step   Muon on shape buckets of 2-D hidden matrices: sum-form momentum,
 *                  Nesterov input, Frobenius normalisation, quintic Newton-Schulz
 *                  orthogonalisation in bf16 on the matrix cores, shape scale and
 *                  decoupled (optionally cautious) weight decay.
 *   ma_adamw_step  the fused elementwise AdamW step over one flat fp32 range
 *                  (embeddings, LM head, normalisation gains, biases).
 *
 * Sources, by page title:
 *   [HB] "Optimizers: AdamW, Muon and the distributed optimizer" (AI infra handbook):
 *        section "AdamW: decoupled weight decay" and section "Muon: orthogonalising
 *        the update" (the update's three steps, the newton_schulz and Muon listings).
 *   [NC] "MuonAdamW vs DistMuonAdamW: Key Differences for Single and Multi-GPU Training
 *        in nanochat": one optimizer with "adamw" and "muon" parameter groups, a fused
 *        AdamW kernel and a fused Muon kernel over same-shape stacks (K, ...).
 *   [DM] "dtensor-muon" package description, "Features" and "Key options": Nesterov
 *        switch, ns_steps, cautious weight decay, decoupled vs coupled Adam decay.
 *   [DMuon] "DMuon: Efficient Distributed Muon Training with Near-Adam Overhead",
 *        section 2.2: batching same-shape matrices, symmetric (lower-triangle) Gram.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  All device memory is owned
 *     by the caller; the library never allocates, frees or keeps a pointer after the
 *     work it enqueued has completed.
 *   - fp32 tensors are contiguous row-major.  Device pointers must be 4-byte aligned;
 *     16-byte alignment (what allocators return) selects the vectorised kernels,
 *     other alignments give identical results through scalar kernels.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).  Calls enqueue
 *     their kernels on it and return without synchronising.
 *   - Argument errors are detected on the host before anything is launched; the
 *     call then returns a negative ma_status and ma_last_error() describes it.
 *     A failed launch returns MA_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.  No C++ exception crosses this boundary.
 *   - Calls are thread-safe with respect to each other as long as they do not share
 *     buffers; ma_last_error() is per calling thread.
 */
#ifndef MUON_ADAMW_H
#define MUON_ADAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MA_ABI_VERSION 4

typedef enum {
  MA_OK = 0,
  MA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad hyperparameter, overlap */
  MA_ERR_UNSUPPORTED = -2, /* valid request outside what this build handles */
  MA_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small */
  MA_ERR_HIP = -4,         /* a HIP runtime call or launch failed */
  MA_ERR_INTERNAL = -5     /* ma_muon_check_plan found a launch that breaks its plan */
} ma_status;

/* One shape bucket of Muon matrices [NC]: K matrices of A x B, stacked (K, A, B).
 * K == 0 is an empty bucket (skipped).  The three buffers must not overlap. */
typedef struct {
  int64_t K, A, B;
  float* param;       /* device, (K, A, B) fp32, updated in place */
  const float* grad;  /* device, (K, A, B) fp32, read only */
  float* momentum;    /* device, (K, A, B) fp32, updated in place; zeros before step 1 */
} ma_muon_bucket;

/* Muon hyperparameters ([HB] update steps; [DM] "Key options"). */
typedef struct {
  float lr;               /* learning rate eta */
  float momentum;         /* mu; M <- mu M + G */
  float weight_decay;     /* lambda; P <- P (1 - eta lambda) before the update */
  float ns_eps;           /* added to ||U||_F before dividing (1e-7 in [HB]) */
  int32_t nesterov;       /* 1: NS input U = G + mu M (new M); 0: U = M */
  int32_t cautious_wd;    /* 1: decay only where update * param > 0 [DM] */
  int32_t ns_steps;       /* Newton-Schulz iterations, 0..MA_MAX_NS_STEPS */
  int32_t scale_mode;     /* 0: 0.2 sqrt(max(A,B)) [HB]; 1: sqrt(max(1, A/B)) [HB] */
  const float* ns_coeffs; /* host, ns_steps x 3 (a, b, c) per iteration; NULL selects
                             the quintic (3.4445, -4.7750, 2.0315) for every iteration */
  int32_t ns_mode;        /* 0: the iteration as printed [HB] (default).
                             1: Gram-space iteration ([DMuon] section 2.2) for buckets
                             whose long side is at least 3.5x the Gram side, in either
                             orientation (others as 0, reported in
                             ma_muon_route.ns_mode_run): R0 = X0 X0^T once, then per step
                             P = a I + b R + c R^2, Q <- P Q, R <- P R P on m x m matrices
                             (m the Gram side), and X = Q X0 at the end: 3 m^2 n +
                             (4 N - 3) m^3 instead of N (3 m^2 n + m^3) FLOP for N steps
                             (symmetric counts; 2.1x fewer at n = 3.5 m and N = 5).  Exact
                             in real arithmetic; R holds squared singular values, so the
                             route runs on fp16 operands (three more significand bits
                             than bf16, same MFMA rate, fp32 accumulation) scaled by
                             powers of two into fp16's range, and returns bf16.  Its error
                             was measured at 2-7e-3 against the exact iteration on
                             Gaussian, low-rank, row-scaled and condition-1e4 gradients at
                             the workloads' sizes, at most 1.3e-2 on small conditioned
                             ones (the printed iteration's bf16 path: 7-10e-3).  Taken only
                             when the coefficients keep every stored value inside fp16
                             (the quintic: up to 8 steps, since Q grows as a^N on a zero
                             singular value); else the bucket runs as under 0. */
} ma_muon_hparams;

#define MA_MAX_NS_STEPS 64

/* Routing report for one bucket (integer, exact).  [HB] newton_schulz listing: a
 * matrix with more rows than columns (A > B, strict) is orthogonalised transposed,
 * so that the Gram matrix X X^T is the smaller square.  m = min(A,B), n = max(A,B).
 * m_pad / n_pad are the tile-padded sizes of the workspace layout. */
typedef struct {
  int32_t transposed;
  int32_t m, n;
  int32_t ns_steps_run;
  int32_t m_pad, n_pad;
  int32_t ns_mode_run;  /* 1 when the bucket runs the Gram-space iteration */
} ma_muon_route;

/* AdamW hyperparameters ([HB] "AdamW: decoupled weight decay"; [DM] is_adamw). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;          /* t >= 1, used for the bias corrections 1 - beta^t */
  int32_t decoupled;     /* 1: AdamW, decay applied to the weights; 0: Adam + L2 */
  int32_t cautious_wd;   /* 1 (decoupled only): decay only where update * param > 0 */
} ma_adamw_hparams;

/* ABI version of the loaded library (MA_ABI_VERSION it was built with). */
int ma_abi_version(void);

/* Static text for a status code. */
const char* ma_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* ma_last_error(void);

/* Host only: the route one A x B matrix takes (see ma_muon_route) under hp->ns_steps and
 * hp->ns_mode.  hp may be NULL (ns_steps 5, ns_mode 0).  Returns MA_ERR_INVALID_ARG for
 * A < 1, B < 1 or a NULL out. */
ma_status ma_muon_route_of(int64_t A, int64_t B, const ma_muon_hparams* hp, ma_muon_route* out);

/* Host only: workspace bytes ma_muon_step needs for these buckets.  Buckets run in
 * phases: consecutive buckets with the same GEMM configuration (tile size and operand
 * layout, fixed by the bucket's shape), at most 4 of them and 4 GiB of workspace
 * together, share each Newton-Schulz launch; a phase of small-tile buckets whose large
 * tiles fill the GPU together is planned on large tiles (its buckets' m_pad / n_pad,
 * and so the need, follow).  The result is the maximum over phases of the phase's
 * summed need.  0 when there is nothing to do, and for invalid arguments (ma_muon_step
 * then reports them). */
size_t ma_muon_workspace_bytes(const ma_muon_bucket* buckets, int32_t n_buckets,
                               const ma_muon_hparams* hp);

/* Host only: how ma_muon_step groups the buckets (the phases of
 * ma_muon_workspace_bytes) under hp->ns_mode (hp may be NULL: ns_mode 0).  Each phase of
 * the printed iteration runs 3 x ns_steps Newton-Schulz GEMM launches (Gram, polynomial,
 * combine per iteration) covering all of its buckets; Gram-space buckets form phases of
 * their own.  Returns the number of phases, or a negative ma_status for invalid
 * arguments (NULL buckets with n_buckets > 0, n_buckets < 0, K < 0, A or B < 1 with
 * K > 0).  phase_of: host, NULL or n_buckets entries, receives each bucket's phase index
 * (-1 for an empty bucket). */
int32_t ma_muon_phases(const ma_muon_bucket* buckets, int32_t n_buckets,
                       const ma_muon_hparams* hp, int32_t* phase_of);

/* One Muon step on every bucket [HB], in this order per bucket:
 *   M <- mu M + G;  U <- G + mu M (nesterov) or M;  X0 <- U / (||U||_F + ns_eps)  (bf16,
 *   transposed when A > B);  ns_steps times: R <- X X^T, P <- a I + b R + c R R,
 *   X <- P X  (= a X + (b R + c R R) X; bf16 operands, fp32 accumulation);
 *   O <- X (un-transposed);
 *   s <- scale(A, B);  P <- P - eta lambda [mask] P - eta s O,
 *   mask = (s O * P > 0) when cautious_wd, else 1.
 * Range: any finite fp32 gradients and momenta whose sum mu M + G stays finite.  ||U||_F
 * is summed in fp64, and a matrix whose norm lies outside [2^-32, 2^32] has its bf16 copy
 * multiplied by a power of two before the first product (exact), so the fp32
 * accumulation of the first Gram product neither overflows nor loses its small terms.
 * NaN or Inf in a matrix's gradient makes that matrix's update non-finite (no scrubbing).
 * buckets:    host array of n_buckets descriptors (n_buckets >= 0).
 * workspace:  device, 256-byte aligned, at least ma_muon_workspace_bytes(...) bytes;
 *             may be NULL when that is 0.  Its contents are scratch.
 * route_out:  host, NULL or an array of n_buckets reports filled before any launch.
 * Errors: MA_ERR_INVALID_ARG (null/overlapping buffers, K < 0, A or B < 1 with K > 0,
 * ns_steps out of range, non-finite hyperparameters), MA_ERR_WORKSPACE, MA_ERR_HIP. */
ma_status ma_muon_step(const ma_muon_bucket* buckets, int32_t n_buckets,
                       const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                       void* stream, ma_muon_route* route_out);

/* One AdamW step over n elements [HB]:
 *   decoupled: p <- p (1 - lr wd)   (cautious: only where update * p > 0)
 *   coupled:   g <- g + wd p
 *   m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *   p <- p - lr mhat / (sqrt(vhat) + eps),  mhat = m / (1 - b1^t),  vhat = v / (1 - b2^t)
 * param, exp_avg, exp_avg_sq are updated in place; grad is read only.  n == 0 is a
 * no-op.  The four ranges must not overlap.
 * Errors: MA_ERR_INVALID_ARG (null pointers with n > 0, n < 0, step < 1, overlap,
 * non-finite hyperparameters), MA_ERR_HIP. */
ma_status ma_adamw_step(float* param, const float* grad, float* exp_avg, float* exp_avg_sq,
                        int64_t n, const ma_adamw_hparams* hp, void* stream);

/* A benchmark aid: the bandwidth ceiling of an elementwise access pattern.  Streams
 * `reads` fp32 arrays in (1..4) and `writes` out (0..3), n elements each (n % 4 == 0,
 * every array 16-byte aligned; an output may be exactly one of the inputs, streamed in
 * place, other overlaps are rejected), with the access pattern of the AdamW
 * kernel (float4 groups, non-temporal loads and stores, four groups per thread) and no
 * other arithmetic: out[j] = in[0] + ... + in[reads-1] + j.  reads = 4, writes = 3 is
 * the AdamW step's pattern (28 bytes per element).  in, out: host arrays of device
 * pointers.  Errors: MA_ERR_INVALID_ARG, MA_ERR_HIP. */
ma_status ma_stream_probe(const float* const* in, int32_t reads, float* const* out,
                          int32_t writes, int64_t n, void* stream);

/* A benchmark aid: the matrix cores' sustained rate on given operand data.  Launches
 * `blocks` blocks of 8 waves (512 threads; with one block per compute unit that is two
 * waves per SIMD, the Newton-Schulz GEMM kernel's occupancy).  Each wave reads 8 A and 8 B
 * operand fragments once from `operands` (device, 16 x 64 x 8 bf16 values = 16 KiB,
 * 16-byte aligned: fragment f of lane l is the 8 values at (f * 64 + l) * 8, A fragments
 * even f, B fragments odd f) and then runs `iters` rounds of 8 v_mfma_f32_32x32x16_bf16,
 * round r pairing A fragment r with B fragment (r + 3) % 8, into four accumulators, with no
 * memory access inside the loop: blocks * 8 * iters * 8 * 32768 FLOP in all.  out (device,
 * blocks * 512 floats, 4-byte aligned) receives each thread's sum of its accumulator
 * elements, so the summed products can be checked.  clocks (device, 2 * blocks values,
 * 8-byte aligned, or NULL) receives per block the shader-clock counter's advance over the
 * loop (s_memtime) and the 100 MHz real-time counter's (s_memrealtime): their ratio times
 * 0.1 GHz is the clock the loop ran at.  The part lowers its clock under sustained MFMA load
 * when the operands toggle, so this rate, not the 2.5 PFLOP/s rating, bounds what any
 * bf16 GEMM reaches on such data.  Errors: MA_ERR_INVALID_ARG (NULL or misaligned
 * pointers, blocks outside 1..65535, iters outside 1..2^22), MA_ERR_HIP. */
ma_status ma_mfma_probe(const void* operands, int32_t blocks, int32_t iters, float* out,
                        uint64_t* clocks, void* stream);

/* One AdamW tensor of ma_adamw_step_multi: n fp32 elements at each pointer (device). */
typedef struct {
  float* param;
  const float* grad;
  float* exp_avg;
  float* exp_avg_sq;
  int64_t n;
} ma_adamw_segment;

/* ma_adamw_step over many tensors at once ([NC]: one fused AdamW over the optimizer's
 * AdamW parameters): segs is a host array of n_segs segments, each updated exactly as
 * ma_adamw_step would (bitwise the same results), in one launch per 48 segments instead of
 * one per tensor.  Segments with n == 0 are skipped.  No written range (param, exp_avg,
 * exp_avg_sq) may overlap any other range of any segment; gradients may be shared.
 * Errors: MA_ERR_INVALID_ARG (as ma_adamw_step, per segment, plus n_segs < 0, segs NULL
 * with n_segs > 0, overlap between segments), MA_ERR_UNSUPPORTED (a segment above 2^31
 * blocks of 4096 elements), MA_ERR_HIP. */
ma_status ma_adamw_step_multi(const ma_adamw_segment* segs, int32_t n_segs,
                              const ma_adamw_hparams* hp, void* stream);

/* Host only: workspace bytes ma_newton_schulz needs for a (K, A, B) stack. */
size_t ma_newton_schulz_workspace_bytes(int64_t K, int64_t A, int64_t B);

/* The orthogonalisation alone ([HB] newton_schulz): for each of K matrices,
 * out = NS(in) in the input's own orientation, fp32, using hp->ns_eps, hp->ns_steps
 * and hp->ns_coeffs (other fields ignored).  in and out must not overlap.
 * Errors: as ma_muon_step. */
ma_status ma_newton_schulz(const float* in, float* out, int64_t K, int64_t A, int64_t B,
                           const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Per-shape GEMM tiles for the Newton-Schulz products ([DMuon] section 2.4: autotuning
 * per shape, cached).  For each phase of the bucket list (ma_muon_phases), the Gram,
 * polynomial and combine launches can run 256 x 256 or 128 x 128 tiles when the phase
 * is planned on 256-tiles (128 only, otherwise; the combine of a phase whose Gram side
 * exceeds 2048 only its 256-tile configuration).  Every choice accumulates each output
 * over the same k order, so results are bitwise the same; only the time differs.
 *   reps > 0: time every available tile of each product (one warm-up launch, then reps
 *             launches between two HIP events on `stream`) on the phase's operands in
 *             the workspace, whose contents are scratch and are overwritten; keep the
 *             fastest.  This call SYNCHRONISES with `stream` (per product and tile) and
 *             creates two HIP events; it launches only GEMMs: parameters, gradients and
 *             momenta are not touched and their pointers may be NULL.
 *   reps = 0: pin the tiles given in `tiles` (0: back to the default rule).
 * tiles:  host, 3 x (number of phases) entries (Gram, polynomial, combine per phase):
 *         output with reps > 0 (may be NULL), input with reps = 0.
 * hp:     may be NULL (the quintic's coefficients are used for the timed polynomial).
 * The chosen tiles are kept for this process, keyed by the phase's shapes, and used by
 * every later ma_muon_step / ma_newton_schulz call whose phase has those shapes.
 * Errors: MA_ERR_INVALID_ARG (bad shapes, reps outside [0, 1000], tiles NULL with
 * reps = 0, a pinned tile the phase cannot run), MA_ERR_WORKSPACE (reps > 0),
 * MA_ERR_HIP. */
ma_status ma_muon_tune(const ma_muon_bucket* buckets, int32_t n_buckets,
                       const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                       void* stream, int32_t reps, int32_t* tiles);

/* The GEMM configuration of one Newton-Schulz product of a phase ([DMuon] section 2.4:
 * tile shape, pipeline configuration, tile order).  A field at its default (0, or -1 for
 * spread) takes the library's rule for it.  Every configuration accumulates each output
 * over the same k order, so results are bitwise the same; only the time differs. */
typedef struct {
  int32_t tile;      /* 128 or 256 (on a 256-padded phase); 192 (combine, Gram sides padded
                        to a multiple of 192); 0: the phase's rule */
  int32_t band;      /* row panels per L2 band of the tile order, 1..64; 0: 4 (8 for a
                        combine whose matrices the XCDs share, xcd 3) */
  int32_t spread;    /* 256- and 192-tiles: 1 spreads the next stage's operand loads over
                        half a stage, 0 issues them at once; -1: 1 */
  int32_t pipeline;  /* 256-tiles of the Gram, the polynomial and the combine of a phase
                        that keeps X^T: 1 = stages of k = 64 in a ring of 3 A and 2 B
                        stages, 2 = four stages of k = 32; 0: 1 */
  int32_t xcd;       /* block order across the 8 XCDs: 1 = each XCD takes a contiguous run
                        of tiles (so its L2 serves neighbouring tiles), 2 = the hardware's
                        round-robin order, 3 = the XCDs share each matrix (XCD x takes the
                        x-th eighth of every matrix's tiles, so the operand panels one
                        XCD misses in its L2 are likely in the memory-side cache from
                        another); 0: 3 for matrices of at least 512 tiles, else 1 */
} ma_gemm_config;

/* ma_muon_tune over whole configurations.  reps > 0: for each product of each phase,
 * search one dimension at a time from the defaults -- tile, then pipeline (where the
 * tile has a choice), then band width (2, 4, 8), then spreading, then the XCD order (1, 2, 3) --
 * timing each candidate
 * as ma_muon_tune does; a candidate replaces the kept one only when at least 3 % faster.
 * The result is reported in configs (host, 3 entries per phase: Gram, polynomial,
 * combine; may be NULL).  SYNCHRONISES, as ma_muon_tune.  When every bucket of a phase
 * gives its gradient pointer, the gradients are first cast into the workspace as
 * ma_muon_step casts them (read only), so the candidates are timed on real operands: the
 * matrix cores' power draw, and with it the clock, depends on the data.
 * reps = 0: pin the given configs (all-default entries of a phase: back to the rules).
 * Errors: as ma_muon_tune (a pinned configuration the phase cannot run:
 * MA_ERR_INVALID_ARG). */
ma_status ma_muon_tune_configs(const ma_muon_bucket* buckets, int32_t n_buckets,
                               const ma_muon_hparams* hp, void* workspace,
                               size_t workspace_bytes, void* stream, int32_t reps,
                               ma_gemm_config* configs);

/* Host only: forget every tuned or pinned configuration (back to the default rules). */
void ma_muon_tune_reset(void);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ma_muon_step with the library's own
 * static workspace of MA_STATIC_WORKSPACE_BYTES instead of a caller workspace.  The
 * workspace is a file-scope device array; each GPU holds its own copy from the first
 * use on that device until the process ends.  Nothing is allocated or freed by these
 * calls; parameters, gradients and momenta are still the caller's.
 *
 * ma_muon_static_init: resolves the current device's copy (hipGetSymbolAddress); called
 * by ma_muon_step_static on its first use on a device.  Call it once per device before
 * capturing a graph that contains ma_muon_step_static.
 * ma_muon_step_static: exactly ma_muon_step (same kernels, same results bit for bit) on
 * the current device's static workspace.  Buckets needing more than
 * MA_STATIC_WORKSPACE_BYTES (ma_muon_workspace_bytes) are rejected with
 * MA_ERR_WORKSPACE before anything is launched.  Every call on one GPU shares that GPU's
 * workspace: calls that overlap on one GPU (other streams, other threads) RACE and must
 * be serialised by the caller; each step rewrites every workspace byte it reads, so
 * nothing needs clearing between calls.
 * Errors: as ma_muon_step, MA_ERR_UNSUPPORTED (device index above 63), MA_ERR_HIP. */
#define MA_STATIC_WORKSPACE_BYTES ((size_t)512 << 20)
ma_status ma_muon_static_init(void);
ma_status ma_muon_step_static(const ma_muon_bucket* buckets, int32_t n_buckets,
                              const ma_muon_hparams* hp, void* stream,
                              ma_muon_route* route_out);

/* What ma_muon_check_plan replayed. */
typedef struct {
  int64_t launches;     /* kernel launches of the step (or of the orthogonalisation) */
  int64_t gemm_blocks;  /* Newton-Schulz GEMM blocks enumerated (padding blocks excluded) */
  int64_t gemm_tiles;   /* output tiles those blocks cover */
} ma_plan_report;

/* Host only: a dry run of every launch ma_muon_step (what = 0) or ma_newton_schulz
 * (what = 1, bucket 0 alone) would enqueue for buckets of these shapes under hp and the
 * tiles this process has tuned or pinned.  The pointers in `buckets` are ignored: the
 * run uses synthetic addresses and touches no GPU.  Every block of every Newton-Schulz
 * GEMM launch is mapped to its output tile by the kernel's own block-to-tile function;
 * its operand reads and result writes must lie inside the workspace buffer (or caller
 * tensor) its argument addresses, and each output tile of a launch must be computed
 * exactly once.  The elementwise launches (cast, norm, rescale, update) are checked the
 * same way.  out (host, may be NULL) receives counts of what was checked.
 * Errors: MA_ERR_INVALID_ARG (what ma_muon_step would reject), MA_ERR_INTERNAL (a launch
 * that breaks the plan; ma_last_error() names it). */
ma_status ma_muon_check_plan(const ma_muon_bucket* buckets, int32_t n_buckets,
                             const ma_muon_hparams* hp, int32_t what, ma_plan_report* out);

/* A benchmark aid: the time of the Newton-Schulz GEMM launches of ma_muon_step, measured
 * on the device.  For each phase (ma_muon_phases) and each of `reps` repetitions, the
 * phase's buckets are cast from their gradients into the workspace as ma_muon_step
 * would (U = G: gradients are read only; parameters and momenta are not touched and may
 * be NULL), then the phase's Newton-Schulz launches run between two HIP events on
 * `stream`.  phase_ms (host, one entry per phase) receives the mean milliseconds per
 * repetition.  This call SYNCHRONISES with `stream` and creates two HIP events.
 * Errors: MA_ERR_INVALID_ARG (shapes, hp, NULL gradients, reps outside [1, 1000], NULL
 * phase_ms), MA_ERR_WORKSPACE, MA_ERR_HIP. */
ma_status ma_muon_ns_time(const ma_muon_bucket* buckets, int32_t n_buckets,
                          const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes,
                          void* stream, int32_t reps, float* phase_ms);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ADAMW_H */
