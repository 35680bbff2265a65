/*
 * sfa.h - C ABI of the sparse fixed-offset attention library (libsfa.so).
 *
 * Causal sparse attention in which query i attends to a dense local window
 * of distances 0..W plus a list of relative offsets shared by all queries,
 * each offset gathered by linear interpolation between two rows of the
 * rotary-rotated keys (and plain values); plus attention over per-query
 * edge lists.  Hand-written HIP kernels for gfx950 (MI355X).
 *
 * Sources, cited by page title and part:
 *   [P1] "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static
 *        Schedules Beat Learned Dilation and Extrapolate Where Dense
 *        Attention Fails" - key-set definition, fib equation, gather
 *        paragraph, alpha parameterisation, schedule list, power-of-2
 *        control, numerical-path paragraph, architecture paragraph.
 *   [P2] "Critical power-law sparse attention" - items 1 and 2.
 *   [P3] "Christoffel-Balanced Sparse Attention" - construction, pseudocode
 *        and production note.
 *
 * Conventions shared by every entry point:
 *   - Every function returns int (or size_t where stated).  >= 0 is success
 *     (producers return the number of entries written), < 0 is an SFA_ERR_*
 *     code.  No function throws, aborts or prints.  sfa_last_error() returns
 *     a thread-local message describing the most recent failure.
 *   - Argument validation is complete before any HIP call: an invalid
 *     argument never touches the device.
 *   - Host producers are pure, synchronous, deterministic and thread-safe;
 *     the caller owns every buffer.
 *   - Device entry points take device pointers allocated by the caller and
 *     enqueue work on `stream` (a hipStream_t, NULL = default stream); they
 *     allocate no memory and return before the work completes.  Errors
 *     raised while the kernels execute surface at the caller's next
 *     synchronisation of that stream.  Calls on different streams are
 *     independent; the library keeps no per-call state.
 *   - Tensor layouts are dense row-major: Q, O, dO, dQ are [B, n, Hq, D];
 *     K, V, dK, dV are [B, n, Hkv, D]; LSE is float [B, Hq, n].  Device
 *     pointers must be 16-byte aligned.  Query head h uses key/value head
 *     h / (Hq / Hkv) (grouped-query attention, [P1] architecture paragraph).
 */
#ifndef SFA_H
#define SFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFA_OK 0
#define SFA_ERR_ARG (-1)         /* null pointer, bad shape, NaN, misalignment */
#define SFA_ERR_CAPACITY (-2)    /* caller buffer too small */
#define SFA_ERR_UNSUPPORTED (-3) /* valid but not built: head_dim, group size, slots */
#define SFA_ERR_HIP (-4)         /* HIP runtime or launch failure */

#define SFA_F32 0  /* float32 tensors */
#define SFA_BF16 1 /* bfloat16 tensors (accumulation is float32) */
/*
 * With SFA_BF16 the forward and the key pass take their products on f16
 * operands: the staged K and V rows (K rotated), the scaled query, the staged
 * rows of the key pass and its probability weights are rounded to f16, and
 * every sum is accumulated in float32 (the query pass and the offset gradient
 * use float32 operands).  Inputs must therefore lie within f16's range:
 * the largest magnitude of each of Q, K, V and dO at most SFA_BF16_MAX_ABS
 * (65504 / sqrt 2, as a rotation can grow one element of a pair by up to
 * sqrt 2) and, unless the tensor is all zeros, at least SFA_BF16_MIN_ABS
 * (2^-14, the smallest normal f16: a tensor wholly below it keeps only f16's
 * subnormal precision).  The kernels do not test this, as a scan costs a
 * pass over every input; sfa_absmax is that scan, for callers who cannot
 * vouch for their inputs, and a tensor outside the range must not be given
 * to the bf16 kernels (larger inputs give non-finite outputs).  Products of
 * in-range inputs need no such care: the key pass scales its f16 dS weights
 * by a power of two taken from a bound the query pass records, so small dO
 * and V together do not push them below f16's normal range.
 */
#define SFA_BF16_MAX_ABS 46318.0f
#define SFA_BF16_MIN_ABS 6.103515625e-05f

#define SFA_MAX_OFFSETS 256 /* shared offsets per call (page 3's m = 128, k = 1024 made bidirectional) */
#define SFA_MAX_SLOTS 320   /* window + 1 + offsets */
#define SFA_MAX_EDGE_WIDTH 256

#define SFA_SCHEDULE_FIXED 0
#define SFA_SCHEDULE_LINEAR 1
#define SFA_SCHEDULE_COPRIME 2

/* Thread-local description of the last error ("" if none). */
const char* sfa_last_error(void);

/* ABI version, currently 1. */
int sfa_version(void);

/* ------------------------------------------------------------------ */
/* Host producers                                                       */
/* ------------------------------------------------------------------ */

/*
 * Rung base of [P1] fib equation: writes 1, 2, 3, 5, ..., 987 (15 entries).
 * Returns 15, or SFA_ERR_CAPACITY if cap < 15, SFA_ERR_ARG if base is NULL.
 */
int sfa_base_fib(int32_t* base, int cap);

/*
 * Reach-matched power-of-2 control base of [P1] (power-of-2 control):
 * writes 2^0 .. 2^10 (11 entries; 1024 matches the Fibonacci reach 987).
 * Returns 11 or an error as sfa_base_fib.
 */
int sfa_base_pow2(int32_t* base, int cap);

/*
 * Scaled rungs of [P1] gather paragraph: d_k = alpha * base[k] (one fp64
 * rounding), lo[k] = floor(d_k), frac[k] = (float)(d_k - lo[k]).  Row pair
 * of query i is i - lo[k] (weight 1 - frac) and i - lo[k] - 1 (weight frac).
 * alpha must be finite and > 0, base[k] >= 0, d_k < 2^30.  Returns k_count,
 * SFA_ERR_ARG on a bad argument.  lo and frac hold k_count entries.
 */
int sfa_offsets_scaled(const int32_t* base, int k_count, double alpha,
                       int32_t* lo, float* frac);

/* sfa_offsets_scaled over the Fibonacci base; returns 15 (cap >= 15). */
int sfa_offsets_fib(double alpha, int32_t* lo, float* frac, int cap);

/* sfa_offsets_scaled over the power-of-2 base; returns 11 (cap >= 11). */
int sfa_offsets_pow2(double alpha, int32_t* lo, float* frac, int cap);

/*
 * Per-layer alpha of the [P1] schedule list.  schedule: SFA_SCHEDULE_FIXED
 * (alpha = 1), SFA_SCHEDULE_LINEAR (alpha = 0.5 + layer/(L-1), computed as
 * the single fp64 division (2 layer + L - 1) / (2 (L - 1))) or
 * SFA_SCHEDULE_COPRIME (the linear value of index (S * layer) mod L; S must
 * be coprime with L).  Requires L >= 2 and 0 <= layer < L.  Writes *alpha,
 * returns SFA_OK or SFA_ERR_ARG.
 */
int sfa_stagger_alpha(int schedule, int layer, int L, int S, double* alpha);

/*
 * alpha = 0.5 + sigmoid(theta) and its derivative (alpha - 1/2)(3/2 - alpha)
 * ([P1] alpha parameterisation).  Either output may be NULL.
 */
int sfa_alpha_of_theta(double theta, double* alpha, double* dalpha_dtheta);

/*
 * Christoffel offsets of [P3] construction: c[j] = floor((j+1)m/k) -
 * floor(jm/k) in 64-bit integer arithmetic for j = 0..k-1; writes the
 * positions j with c[j] == 1 in ascending order (exactly m of them).  Used
 * as backward distances by the causal kernel (row i - o).  Requires
 * 1 <= k <= 2^24, 0 <= m <= k.  Returns m, SFA_ERR_CAPACITY if cap < m.
 */
int sfa_offsets_christoffel(int m, int k, int32_t* offsets, int cap);

/*
 * Bidirectional Christoffel offsets ([P3], signed offsets): -O and +O of
 * sfa_offsets_christoffel, ascending (2m values), for a layer run with
 * SFA_FLAG_SIGNED_OFFSETS.  Same requirements; returns 2m,
 * SFA_ERR_CAPACITY if cap < 2m.
 */
int sfa_offsets_christoffel_signed(int m, int k, int32_t* offsets, int cap);

/*
 * Power-law edge lists of [P2] items 1-2.  For query i: the window
 * {i-r..i+r} clipped to [0, n), plus `draws` keys j = (i + s d) mod n with
 * d ~ q(d) = d^-(1+sigma) / sum_{u <= n/2} u^-(1+sigma) and a random sign s;
 * union, ascending, padded with -1 to `width`.  Randomness: SplitMix64,
 * key_i = mix(seed ^ mix(i)), draw t uses mix(key_i + 2t) for the distance
 * (u = top 53 bits / 2^53, smallest d with u < CDF[d], CDF accumulated in
 * increasing d in fp64 and normalised, last entry 1) and mix(key_i + 2t + 1)
 * for the sign (top bit 0 -> +1).  edges is int32 [n][width], count int32
 * [n].  Requires n >= 2, r >= 0, draws >= 0, sigma finite and > -1,
 * width <= SFA_MAX_EDGE_WIDTH.  Returns the largest count, or
 * SFA_ERR_CAPACITY if some list exceeds width (buffers then undefined).
 */
int sfa_edges_powerlaw(int n, int r, double sigma, int draws, int width,
                       uint64_t seed, int32_t* edges, int32_t* count);

/*
 * Inverted edge table for the edge-list backward (key-side gather): pages
 * 2 and 3 propose training with these masks ([P2] item 4, [P3]).  For every
 * key j, inv[j][0..inv_count[j]) lists the slots s = i * width + t with
 * t < count[i] and edges[i][t] = j, in ascending order (-1 padded to cap).
 * edges/count as produced by sfa_edges_powerlaw (host, int32 [n][width] and
 * [n]); every listed key must lie in [0, n).  inv == NULL: returns the cap
 * needed (largest in-degree, at least 1) without writing.  Otherwise inv is
 * int32 [n][cap] and inv_count int32 [n], both caller-owned; returns the cap
 * needed, or SFA_ERR_CAPACITY if cap is smaller, SFA_ERR_ARG on bad input.
 */
int sfa_edges_transpose(int n, int width, const int32_t* edges, const int32_t* count, int cap, int32_t* inv,
                        int32_t* inv_count);

/*
 * Rotary table of [P1] gather and architecture paragraphs (Su et al.
 * rotation of interleaved pairs): table[m][p][0] = cos(m * theta^(-2p/D)),
 * table[m][p][1] = sin(...), computed in fp64 and stored as float, for
 * m = 0..n-1 and p = 0..D/2-1.  Requires n >= 1, even head_dim >= 2,
 * theta > 0.  Returns SFA_OK.  The caller copies it to the device and passes
 * it as sfa_attn.rope.
 */
int sfa_rope_table(int n, int head_dim, double theta, float* table);

/* ------------------------------------------------------------------ */
/* Device attention                                                     */
/* ------------------------------------------------------------------ */

/*
 * Largest magnitude of a device tensor, for the bf16 range check (see
 * SFA_BF16): folds the IEEE bits of max |x| over the count elements of x
 * (dtype SFA_F32 or SFA_BF16, 16-byte aligned) into the device word *result
 * (4-byte aligned, caller-owned, cleared by the caller) with an atomic
 * maximum.  Read as a float, *result is the largest magnitude, +inf if some
 * element is infinite and NaN if some element is NaN.  Asynchronous on
 * `stream`.  Returns SFA_OK, SFA_ERR_ARG on a bad argument (before any HIP
 * call) or SFA_ERR_HIP.
 */
int sfa_absmax(const void* x, int64_t count, int dtype, uint32_t* result,
               void* stream);

/*
 * sfa_attn.flags.  SFA_FLAG_INTERP_KERNEL: sfa_fwd runs the interpolating
 * instantiation of the shared-offset kernel even when every offset is an
 * integer (frac == 0 everywhere).  By default such a layer runs the integer
 * instantiation, which has no interpolation code: the pages' fused
 * integer-offset kernel against their learned interpolated gather
 * ("Depth-Staggered Fibonacci Spacing for Sparse Attention", results
 * discussion of the learned variant).  Both give bit-identical results; the
 * flag exists to measure and test that.
 */
#define SFA_FLAG_INTERP_KERNEL 1
/*
 * SFA_FLAG_SIGNED_OFFSETS: off_lo may be negative (|off_lo| < 2^30).  A
 * negative offset names the later row i - lo = i + |lo| (and i - lo - 1
 * with weight frac), valid while it is below n: page 3's bidirectional
 * attention by signed offsets ("Christoffel-Balanced Sparse Attention",
 * integration paragraph).  Without the flag every off_lo must be >= 0
 * (causal).  The window slots 0..W stay causal.
 */
#define SFA_FLAG_SIGNED_OFFSETS 2

/*
 * Problem description (plain data; host arrays are read during the call
 * and not retained).
 */
typedef struct sfa_attn {
  int32_t batch;    /* B >= 0 (0 -> nothing to do) */
  int32_t seqlen;   /* n >= 0 */
  int32_t hq;       /* query heads, multiple of hkv */
  int32_t hkv;      /* key/value heads; group size hq/hkv in {1, 2, 4, 8} */
  int32_t head_dim; /* D in {16, 32, 64, 128} (128: bf16 only), D/(hq/hkv) >= 2 */
  int32_t dtype;    /* SFA_F32 or SFA_BF16, for Q, K, V, O, dO, dQ, dK, dV */
  int32_t window;   /* W >= 0: distances 0..W, self always present ([P1]) */
  int32_t n_off;    /* shared offsets, 0..SFA_MAX_OFFSETS */
  float scale;      /* logit scale; 0 -> 1/sqrt(D) ([P2] item 2, [P3]) */
  int32_t flags;    /* SFA_FLAG_* bits, 0 by default */
  const int32_t* off_lo; /* host [n_off]: floor of each offset distance, >= 0
                            (any sign with SFA_FLAG_SIGNED_OFFSETS) */
  const float* off_frac; /* host [n_off]: interpolation weight in [0, 1) */
  const float* rope;     /* device [n][D/2][2] from sfa_rope_table, or NULL
                            for no rotation */
} sfa_attn;

/*
 * Forward over the window and shared offsets ([P1] key set and gather
 * paragraph; [P3] pseudocode for offsets with frac = 0 and window = 0).
 * Slot s <= W of query i is row i - s, valid iff i - s >= 0; offset k is
 * (1 - frac_k) R(i-lo_k) K[i-lo_k] + frac_k R(i-lo_k-1) K[i-lo_k-1] (and the
 * same for V without rotation), valid iff i >= lo_k + frac_k.  Every slot is
 * its own logit (duplicates count twice).  Logits are scale * <R(i) q, k~>,
 * softmax over valid slots, O = sum p v~.  o: output [B, n, Hq, D] in
 * dtype; lse: optional float [B, Hq, n] natural-log sum of exp(logit)
 * (NULL to skip).  Returns SFA_OK or an error; W + 1 + n_off must not exceed
 * SFA_MAX_SLOTS.
 */
int sfa_fwd(const sfa_attn* a, const void* q, const void* k, const void* v,
            void* o, float* lse, void* stream);

/*
 * Forward over per-query edge lists ([P2] item 2; [P3] pseudocode): keys
 * of query i are edges[i][t] for t < count[i] (device int32 [n][width] and
 * [n], shared by all batch entries and heads); entries outside [0, n) are
 * skipped.  No causal filter.  a->window and a->n_off are ignored.  Rotary
 * rotation applies if a->rope is set.  1 <= width <= SFA_MAX_EDGE_WIDTH.
 */
int sfa_fwd_edges(const sfa_attn* a, const int32_t* edges,
                  const int32_t* count, int width, const void* q,
                  const void* k, const void* v, void* o, float* lse,
                  void* stream);

/*
 * Workspace bytes sfa_bwd needs for this problem (0 on invalid arguments;
 * see sfa_last_error).
 */
size_t sfa_bwd_workspace_bytes(const sfa_attn* a);

/*
 * Backward of sfa_fwd for L = <O, dO> ([P1] gather and numerical-path
 * paragraphs: the interpolation carries the gradient to the offsets).
 * Inputs q, k, v, lse (from sfa_fwd of the same problem) and dout.  The
 * forward output itself is not needed: rowsum(dO * O) is recomputed exactly
 * as sum over slots of p * (dO . v~).  Outputs dq [B, n, Hq, D], dk, dv
 * [B, n, Hkv, D] in dtype (overwritten).  dd: optional device float
 * [n_off], dd[k] = dL/dd_k inside the current interpolation cell (the
 * derivative of the row pair: row(i-lo-1) - row(i-lo), taken also when
 * frac = 0), formed from float32 operands and summed in double for either
 * dtype.  dtheta: optional device float scalar, (alpha - 1/2)(3/2 -
 * alpha) * sum_k base[k] dd[k] ([P1] alpha parameterisation); needs base
 * (host int32 [n_off], the unscaled rungs) and alpha.  workspace: device
 * buffer of at least sfa_bwd_workspace_bytes(a) bytes, 16-byte aligned,
 * contents undefined on entry and exit.  Deterministic: no atomics, fixed
 * reduction order.
 */
int sfa_bwd(const sfa_attn* a, const void* q, const void* k, const void* v,
            const float* lse, const void* dout, void* dq, void* dk, void* dv,
            float* dd, const int32_t* base, double alpha, float* dtheta,
            void* workspace, size_t ws_bytes, void* stream);

/*
 * sfa_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * sfa_bwd (bit-identical outputs); the workspace is the library's static
 * device scratch of SFA_NOALLOC_SCRATCH_BYTES, one copy per device, taken
 * when the library's device code is first used on that device and held until
 * the process ends.  Allocates nothing.  A problem whose sfa_bwd_workspace_bytes
 * exceeds SFA_NOALLOC_SCRATCH_BYTES returns SFA_ERR_CAPACITY before any HIP
 * call (the page-1 learned-alpha step, 32 x 1024 tokens at 8/2 heads, needs
 * about 122 MB).  Calls that overlap on one device share the scratch and race:
 * serialise them (one stream, or events).  The first call on a device looks up
 * that device's copy with hipGetSymbolAddress.
 */
#define SFA_NOALLOC_SCRATCH_BYTES (128ull * 1024 * 1024)
int sfa_bwd_noalloc(const sfa_attn* a, const void* q, const void* k, const void* v,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    float* dd, const int32_t* base, double alpha, float* dtheta,
                    void* stream);

/*
 * Backward of sfa_fwd_edges for L = <O, dO> (training with the per-query
 * masks: [P2] item 4, [P3]).  edges/count: the device lists of the forward;
 * inv/inv_count: their transpose from sfa_edges_transpose (device copies of
 * the host output, int32 [n][inv_width] and [n]); inv must be the transpose
 * of exactly these lists.  lse: the forward's [B][Hq][n] log-sum-exp.  Writes
 * dQ (like q), dK, dV (like k) in the input dtype.  Window and offsets of
 * `a` are ignored.  The workspace (device, 16-byte aligned, at least
 * sfa_bwd_edges_workspace_bytes(a, width) bytes) holds p and dp of every
 * slot and Dvec between the two launches.  Deterministic: no atomics, fixed
 * summation order.  Errors as sfa_bwd.
 */
size_t sfa_bwd_edges_workspace_bytes(const sfa_attn* a, int width);
int sfa_bwd_edges(const sfa_attn* a, const int32_t* edges, const int32_t* count, int width,
                  const int32_t* inv, const int32_t* inv_count, int inv_width, const void* q,
                  const void* k, const void* v, const float* lse, const void* dout, void* dq,
                  void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* Kernel timing (measurement support; off by default)                  */
/* ------------------------------------------------------------------ */

/*
 * When enabled, every kernel launch is timed by two HIP events on its launch
 * stream, which the dispatch itself takes as its start and end timestamps
 * (a call that launches one kernel several times re-records the end event
 * after the last launch).  sfa_profile_read synchronises the recorded events
 * and returns the accumulated milliseconds and launch count of the named
 * kernel ("fwd_offsets", "fwd_edges", "bwd_query", "bwd_key",
 * "bwd_edges_query", "bwd_edges_key", "bwd_reduce"; with bf16 tensors the
 * dd reduction runs inside the "bwd_key" launch);
 * sfa_profile_reset drops all records.  sfa_profile_select(name) restricts
 * the recording to the launches of the named kernel (recording every kernel
 * lengthens a step, and each kernel's average reads higher than with that
 * kernel alone selected); sfa_profile_select(NULL) records every kernel again.  Not
 * thread-safe with concurrent launches.
 */
int sfa_profile_enable(int on);
int sfa_profile_select(const char* kernel);
int sfa_profile_read(const char* kernel, double* total_ms, int64_t* launches);
int sfa_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* SFA_H */
