/*
 * muon_ns.h — C ABI of the MI355X (gfx950) Muon / Newton–Schulz library.
 *
 * What is computed (sources are the pages this library implements):
 *   - DMuon technical summary (gist.science, Korean), §1 "Problem definition":
 *     Muon applies a Newton–Schulz (NS) iteration to the momentum-accumulated
 *     gradient of each weight matrix.
 *   - same page, §2.2 "Efficient Gram Newton–Schulz iteration": the iteration
 *     runs in the m×m Gram space G = X·Xᵀ (m < n), exploits the symmetry of G
 *     with SYRK-style upper-triangle products, and batches matrices of similar
 *     shape so that one dispatch serves many of them.
 *   - DeMuon technical summary (gist.science, Korean), Method §1: momentum is
 *     a moving average of gradients and the update applies msgn(·).
 *
 * Per matrix (stored rows × cols, row-major), with m = min(rows, cols):
 *   X₀ = M / (‖M‖_F + eps), transposed first when rows > cols;
 *   s times: A = X·Xᵀ; X ← a·X + (b·A + c·A²)·X   (computed in Gram space);
 *   O = X transposed back to rows × cols.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     owned by the caller.  The library only borrows them for the enqueue.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream), asynchronously: results are valid once the stream reaches
 *     the enqueued work.  No entry point synchronises the host with the GPU.
 *   - Concurrent lanes: a call whose Gram-space products have fewer than
 *     1536 tiles of all its groups (six rounds of the 256 compute units)
 *     and that holds at least two matrices splits its matrices into two
 *     sets of about equal work (three when under 256 tiles in at least three
 *     groups), each running its own passes and whole product chain on its
 *     own stream; the launches are made round-robin across the lanes.  The
 *     extra streams are the library's (default priority, created on the
 *     first such call on a device, never while `stream` is being
 *     captured); they wait for an event recorded on `stream` and
 *     `stream` waits for each of them at the end, so the call is still one
 *     ordered piece of work on `stream` and can be captured into a graph
 *     once they exist (before that, a captured call runs on `stream`
 *     alone).  A matrix's arithmetic does not depend on the split, so the
 *     results are the same bit for bit.  MUON_LANES=1..4 in the environment
 *     fixes the number of lanes.
 *   - `workspace` is caller-allocated device memory of at least the size
 *     the matching *_workspace_size query returns, 256-byte aligned, that
 *     overlaps no tensor of the call (MUON_ERR_ALIAS otherwise).  Its
 *     contents on entry do not matter and are garbage on exit.  Calls that
 *     share a workspace must be ordered (same stream, or synchronised).
 *   - Thread safety: entry points may be called from several threads; the
 *     tile table and the profiling records are process-wide and guarded.
 *     Do not enable profiling while a stream is being captured into a graph
 *     (the event records would be captured too).
 *   - Argument checks run on the host BEFORE any HIP call.  On any error
 *     nothing is enqueued and a status other than MUON_OK is returned; the
 *     message is available from muon_last_error() (per thread).
 *   - NaN / Inf in the inputs propagate to the outputs; nothing is repaired.
 *   - No C++ exception crosses this boundary.
 *   - Debugging: with MUON_DEBUG_SYNC=1 in the environment, every launch is
 *     followed by a synchronisation of its stream and an error check, so a
 *     failing kernel is named in muon_last_error() (not while the stream is
 *     being captured into a graph).  The default is fully asynchronous.
 */
#ifndef MUON_NS_H
#define MUON_NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_NS_ABI_VERSION 7

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad stride, bad scalar */
  MUON_ERR_UNSUPPORTED = 2, /* a valid request the library does not handle  */
  MUON_ERR_ALIAS = 3,       /* writable ranges that overlap                  */
  MUON_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned    */
  MUON_ERR_HIP = 5,         /* a HIP call or kernel launch failed            */
  MUON_ERR_NO_DEVICE = 6    /* no HIP device is visible                      */
} muon_status_t;

typedef enum muon_dtype {
  MUON_DTYPE_F32 = 0,  /* IEEE float32                                   */
  MUON_DTYPE_BF16 = 1  /* bfloat16 (8 significant bits, float32 range)   */
} muon_dtype_t;

/* One matrix of a batched orthogonalisation.
 *   x:    input, rows × cols, element (i, j) at x[i*ld_x + j], dtype of the call
 *   out:  output, same shape and dtype, element (i, j) at out[i*ld_out + j]
 *   rows, cols ≥ 0 (a matrix with no elements is skipped);
 *   ld_x ≥ cols, ld_out ≥ cols (elements).
 * out may equal x (in place): every input is read before any output is
 * written.  Outputs of different matrices must not overlap. */
typedef struct muon_ns_desc {
  const void* x;
  void* out;
  int64_t rows;
  int64_t cols;
  int64_t ld_x;
  int64_t ld_out;
} muon_ns_desc_t;

/* Batched Newton–Schulz orthogonalisation (DMuon summary §2.2: batched Gram
 * NS over matrices of similar shape).
 *
 * For every desc[i]: out = NS_steps(x / (‖x‖_F + eps)), orientation handled
 * internally (rows > cols is processed as its transpose).
 *   count ≥ 0 (0 is a no-op), 0 ≤ steps ≤ 64, coeffs = {a, b, c} finite,
 *   eps ≥ 0 finite.
 * Precision:
 *   MUON_DTYPE_F32:  fp32 MFMA products on fp32 operand copies;
 *   MUON_DTYPE_BF16: half-precision MFMA products (fp16 operands scaled by
 *                    powers of two, fp32 accumulation), with one exception
 *                    and one addition, decided per group of matrices that
 *                    share m (nearly square means n ≤ 2m):
 *                    - m ≤ 1024 and nearly square: the whole recursion runs
 *                      on fp32 operands with fp32 MFMA (small square Gram
 *                      matrices are the worst conditioned);
 *                    - 1024 < m ≤ 2048 and at least one nearly square
 *                      matrix in the group: fp16 operands plus fp32 copies
 *                      of A and P·A (the a·Y terms of the A-chain);
 *                    - every other group (all wide matrices, n > 2m, and
 *                      every m > 2048): fp16 operands only, no fp32 state.
 * The matrices are grouped by shape: one launch per stage serves every
 * matrix of a group. */
muon_status_t muon_ns_batched(const muon_ns_desc_t* desc, int32_t count, int32_t steps,
                              const float coeffs[3], muon_dtype_t dtype, float eps,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch of muon_ns_batched_noalloc (64 MiB per
 * device the library runs on, held from module load until the process
 * ends). */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)

/* muon_ns_batched for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as muon_ns_batched, with
 * no workspace argument: the workspace is a fixed array of
 * MUON_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per
 * device.  Neither this call nor anything it calls allocates device memory
 * (no hipMalloc / hipFree, no allocating library routine), it records no
 * profiling events, and it runs on `stream` alone (no concurrent lanes, so
 * it creates no stream or event either).
 *   - A request whose workspace (muon_ns_workspace_size) exceeds
 *     MUON_NOALLOC_SCRATCH_BYTES returns MUON_ERR_WORKSPACE before any HIP
 *     call; nothing is enqueued.
 *   - Every call on one device uses that device's single scratch array, and
 *     the array keeps the last call's contents (no call relies on its
 *     contents at entry).  Calls that may overlap on one device race: order
 *     them on one stream or synchronise them.
 *   - The first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress) with the device current; later calls reuse it. */
muon_status_t muon_ns_batched_noalloc(const muon_ns_desc_t* desc, int32_t count, int32_t steps,
                                      const float coeffs[3], muon_dtype_t dtype, float eps,
                                      void* stream);

/* Workspace bytes muon_ns_batched needs for this list of matrices (only the
 * rows/cols of desc are read; pointers may be NULL).  Host only. */
muon_status_t muon_ns_workspace_size(const muon_ns_desc_t* desc, int32_t count,
                                     muon_dtype_t dtype, size_t* bytes);

/* One Muon optimiser step over `count` weight matrices (DMuon summary §1 and
 * §2.2; momentum as in DeMuon Method §1), in place:
 *   momentum[i] ← beta·momentum[i] + grads[i]                 (fp32, one FMA)
 *   O           = NS_steps(momentum[i] / (‖momentum[i]‖_F + eps))
 *   params[i]   ← round(params[i] − lr·√max(1, rows/cols)·O)   (RNE to param dtype)
 * Tensors are contiguous row-major rows[i] × cols[i]:
 *   params[i]:   param_dtype (MUON_DTYPE_BF16 or MUON_DTYPE_F32), read + written
 *   grads[i]:    float32, read
 *   momentum[i]: float32, read + written (the optimiser state; the caller
 *                owns it and may save / restore it between steps)
 * rows[i], cols[i] ≥ 0 (empty matrices are skipped), count ≥ 0,
 * 0 ≤ steps ≤ 64, beta, lr, eps finite, eps ≥ 0.  No range among params,
 * grads and momentum may overlap another.  The NS products use the
 * half-precision MFMA path described under muon_ns_batched. */
muon_status_t muon_step(void* const* params, const float* const* grads, float* const* momentum,
                        const int64_t* rows, const int64_t* cols, int32_t count,
                        muon_dtype_t param_dtype, float beta, float lr, int32_t steps,
                        const float coeffs[3], float eps,
                        void* workspace, size_t workspace_bytes, void* stream);

/* An entry of muon_step_opts_t.scale_exp that carries no exponent. */
#define MUON_SCALE_EXP_UNKNOWN INT32_MIN

/* Options of muon_step_ex.  The pages define the plain step only (momentum
 * as above, no weight decay); the first three are the usual Muon-optimiser
 * variants, provided for use as a drop-in optimiser (DMuon summary §3: the
 * module replaces the optimiser without changing the framework); overlap and
 * max_workspace_bytes choose how the work is scheduled and never change a
 * result beyond what the grouping of matrices changes (see below);
 * scale_exp lets the momentum pass write the half-precision operand itself.
 * A zero-initialised struct with grad_dtype = MUON_DTYPE_F32 is the plain
 * step.
 *   nesterov = 1:  the matrix orthogonalised is u = g + beta·M' (M' the
 *                  updated momentum) instead of M'; the stored state is M'.
 *   weight_decay:  decoupled, W ← round((1 − lr·weight_decay)·W − lr·sc·O);
 *                  0 leaves the plain update unchanged.  Finite, ≥ 0.
 *   grad_dtype:    MUON_DTYPE_F32 or MUON_DTYPE_BF16 gradients (momentum
 *                  stays fp32; bf16 values are widened exactly).
 *   overlap = 1:   a call over at least 2^30 elements runs as two chunks of
 *                  the matrix list (in order, 1/4 and 3/4 of the work) whose
 *                  momentum / norm / cast passes run on a stream the library
 *                  owns (one per device, default priority), each chunk's
 *                  products waiting for its passes on `stream`, so the
 *                  passes of the second chunk overlap the products of the
 *                  first.  The call still orders all its work before later
 *                  work on `stream`, and is capturable into a graph once
 *                  the library's stream exists (while `stream` is being
 *                  captured the library does not create it and runs on
 *                  `stream` alone).  0 (and opts NULL): every launch on
 *                  `stream`.  Measured on the 196-matrix Qwen2.5-7B-shaped
 *                  step the overlap gains at most 0.4%: the products slow
 *                  down by nearly as much as the passes they hide.
 *   max_workspace_bytes > 0: a budget.  The matrices are split, in order,
 *                  into consecutive chunks whose workspace fits the budget;
 *                  the chunks run one after another on `stream`, reusing
 *                  one region, so workspace_bytes ≥ the largest chunk's
 *                  need suffices (≤ the budget).  A matrix that alone
 *                  needs more returns MUON_ERR_WORKSPACE.  0: no budget.
 * A matrix's result depends only on the configuration of its Gram group
 * (tile, operand type, fp32 state: see muon_ns_batched), so chunking leaves
 * it bit for bit unchanged unless the split changes that configuration (a
 * group of one m mixing nearly square and wide matrices, or a tile table
 * keyed by batch size). */
typedef struct muon_step_opts {
  int32_t nesterov;          /* 0 or 1 */
  float weight_decay;
  muon_dtype_t grad_dtype;
  int32_t overlap;           /* 0 or 1 */
  uint64_t max_workspace_bytes;
  int32_t* scale_exp;        /* NULL or count int32 on the device (see below) */
} muon_step_opts_t;

/*   scale_exp:     NULL, or device memory of the call's device holding one
 *                  int32 per matrix (count entries, 4-byte aligned, not
 *                  overlapping any tensor of the call or the workspace),
 *                  read and rewritten by the call: the optimiser state of a
 *                  per-matrix power-of-two operand exponent.  Initialise it
 *                  to MUON_SCALE_EXP_UNKNOWN (any value outside [-100, 100]
 *                  means unknown).  With it, matrices on the fp16 256-tile
 *                  path have their momentum pass write the MFMA operand X₀'
 *                  = u·2^e (u the matrix orthogonalised) directly, instead of
 *                  a second pass re-reading the fp32 momentum after the norm;
 *                  the products then use X₀ = ρ·X₀' with ρ = sX/((‖u‖+eps)·2^e)
 *                  applied in fp32 in the SYRK (ρ²) and final-product (ρ)
 *                  epilogues.  X₀' is kept when ‖u‖·2^e ∈ [2^9, 2^14] (no
 *                  fp16 overflow, entries as far from fp16's subnormal range
 *                  as the normalised operand's); otherwise, and when e is
 *                  unknown, the matrix is cast from the momentum as without
 *                  scale_exp.  Each entry is then rewritten to the exponent
 *                  that puts ‖u‖·2^e in [2^12, 2^13) (MUON_SCALE_EXP_UNKNOWN
 *                  when ‖u‖ is 0 or not finite), for the next step.  Results
 *                  agree with the call without scale_exp to the rounding of
 *                  the fp16 operand (the same precision, another scale), not
 *                  bit for bit; ‖u‖ is also summed in another order (per
 *                  64×64 tile), so even a matrix that falls back to the cast
 *                  may differ in the last bits.  Matrices on other paths
 *                  (fp32 groups, 128-tile groups) ignore their entry and
 *                  leave it unchanged. */
/* muon_step with options; opts = NULL gives exactly muon_step.  grads[i]
 * has opts->grad_dtype; every other argument, the workspace size and the
 * error behaviour are those of muon_step (an invalid option returns
 * MUON_ERR_INVALID_ARG before anything is enqueued). */
muon_status_t muon_step_ex(void* const* params, const void* const* grads, float* const* momentum,
                           const int64_t* rows, const int64_t* cols, int32_t count,
                           muon_dtype_t param_dtype, float beta, float lr, int32_t steps,
                           const float coeffs[3], float eps, const muon_step_opts_t* opts,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Row/column-selected Muon step with error feedback, in place.
 * Dion3 review (blog.secrett2633.cloud), §3 "Method & Key Results": the
 * update rule uses only part of the rows / columns of the momentum matrix to
 * shrink the orthogonalisation; §1 "Key Terms & Definitions", Error
 * Feedback: what a reduced-size update leaves out is corrected in later
 * steps.  The page gives no formula; this entry point computes, per matrix
 * (stored rows × cols, m = min(rows, cols)):
 *   B = momentum[i] + grads[i]                                   (fp32 add)
 *   score of each row of the oriented m×n view of B (stored rows when
 *   rows ≤ cols, stored columns when rows > cols) = its squared ℓ2 norm,
 *   summed in fp32; S = the k = max(1, ⌈fraction·m⌉) highest scores (ρ·m
 *   formed in double), equal scores taken lowest index first;
 *   O_S = NS_steps(B_S / (‖B_S‖_F + eps))  on the k×n block (Gram size k);
 *   params[i] rows (columns) in S ← round(W − lr·√max(1, rows/cols)·O_S),
 *   all other weights unchanged bit for bit;
 *   momentum[i] ← β·B on S and B elsewhere (the unused rows are carried at
 *   full weight: error feedback).
 * With fraction = 1 the update equals muon_step's (B then follows
 * B ← β·B + g) and the stored buffer is β·B.
 * Tensors are contiguous row-major: params[i] param_dtype (BF16 or F32),
 * grads[i] float32 (read), momentum[i] float32 (read + written).
 * 0 < fraction ≤ 1 (MUON_ERR_INVALID_ARG otherwise); every other argument,
 * the aliasing rules and the error behaviour are those of muon_step.  The
 * selection is made in fp32 on the GPU: rows whose scores differ by less
 * than fp32 summation error may be selected either way.  The k×n blocks go
 * through the half-precision MFMA pipeline of muon_ns_batched. */
muon_status_t muon_step_selected(void* const* params, const float* const* grads,
                                 float* const* momentum, const int64_t* rows, const int64_t* cols,
                                 int32_t count, muon_dtype_t param_dtype, float beta, float lr,
                                 int32_t steps, const float coeffs[3], float eps, double fraction,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes muon_step_selected needs for these shapes and fraction.
 * Host only. */
muon_status_t muon_step_selected_workspace_size(const int64_t* rows, const int64_t* cols,
                                                int32_t count, double fraction, size_t* bytes);

/* Workspace bytes muon_step (and muon_step_ex without a budget) needs for
 * these shapes, with or without opts->overlap.  Host only. */
muon_status_t muon_step_workspace_size(const int64_t* rows, const int64_t* cols, int32_t count,
                                       size_t* bytes);

/* Writes a JSON description of the launch plan (groups, tile sizes, padded
 * sizes, workspace offsets, operand scales) for these shapes into buf
 * (NUL-terminated, truncated to buf_len).  `for_step` selects the muon_step
 * plan (1) or the muon_ns_batched plan (0, with `dtype`).  Host only; used by
 * tests and tuning tools. */
muon_status_t muon_describe_plan(const int64_t* rows, const int64_t* cols, int32_t count,
                                 int32_t for_step, muon_dtype_t dtype, int32_t steps,
                                 const float coeffs[3], char* buf, size_t buf_len);

/* Tuning table: the launch configuration the planner uses for a Gram group
 * (one m and operand type), keyed by the group's size m, its largest n, its
 * operand type (0: fp16 operands, 1: fp32 operands) and batch-size class
 * floor(log2(number of matrices in the group)).  DMuon summary §2.4 tunes
 * kernel configurations per shape at start-up and keeps them in a cache;
 * `python -m muon_newton_schulz_06_amd.autotune` measures such a table and
 * installs it with this call.  Per entry:
 *   m ≥ 1; n ≥ 0 (0 matches any n; an entry with the group's own n takes
 *   precedence); 0 ≤ count_class ≤ 31;
 *   tile:       128 or 256 for fp16 groups, 32, 64 or 128 for fp32 groups
 *               (32: the contraction split over four waves, the built-in
 *               choice for m ≤ 256), or 0 for the built-in choice;
 *   xcd_window: logical tiles each XCD runs in a row (8, 16, 32 or 64), or 0
 *               for the built-in 32;
 *   band:       tile rows per band of the tile order (1, 2, 4 or 8), or 0
 *               for the built-in 4.
 * At most 4096 entries.  The table replaces the previous one process-wide
 * (n = 0 clears it); groups without an entry use the built-in choices.
 * Groups that carry fp32 A-chain state always use 128-tiles (the tile order
 * still applies).  An invalid entry leaves the table unchanged.  The tile
 * changes the summation order of the products, so results under a table
 * keyed by batch size may differ in the last bits from one batch to another;
 * the tile order changes nothing but the order in which tiles run. */
typedef struct muon_tile_entry {
  int64_t m;
  int64_t n;
  int32_t op;
  int32_t count_class;
  int32_t tile;
  int32_t xcd_window;
  int32_t band;
  int32_t reserved; /* 0 */
} muon_tile_entry_t;

muon_status_t muon_set_tile_table(const muon_tile_entry_t* entries, int32_t n);

/* Kernel-time instrumentation.  While enabled, every launch the library
 * makes is bracketed by a pair of HIP events on the launch's stream and its
 * algorithmic work is recorded.  muon_profile_read waits for the recorded
 * events, returns the totals for one kind and clears that kind's records.
 * Kinds: 0 momentum / sum of squares, 1 norm finish, 2 cast + transpose,
 *        3 SYRK, 4 symmetric Gram-space products on 128×128 tiles,
 *        5 final product + update, 6 Gram-space a·Y + B·Y products on
 *        256×256 tiles, 7 Gram-space A² products on 256×256 tiles,
 *        8 selected step: B = M + g and row scores, 9 its top-k,
 *        10 its gather, 11 its scatter of the update.
 * work is algorithmic flops for kinds 3–7 and algorithmic HBM bytes for the
 * others.  The launches of concurrent lanes overlap in time, so their
 * kernel times add up to more than the call's duration. */
muon_status_t muon_profile_enable(int32_t on);
muon_status_t muon_profile_read(int32_t kind, double* total_ms, int64_t* launches, double* work);

/* Message of the last failed call on this thread ("" if none). */
const char* muon_last_error(void);

/* MUON_NS_ABI_VERSION of the loaded library. */
int32_t muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_NS_H */
