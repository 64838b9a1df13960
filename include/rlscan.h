/*
 * rlscan.h -- C ABI of librlscan: batched first-order linear-recurrence scans
 * for reinforcement-learning credit assignment on AMD Instinct MI355X (gfx950).
 *
 * Every estimator below is one instance of the recurrence
 *     x_t = a_t * x_{t+1} + b_t      (reverse-time estimators)
 *     x_t = a_t * x_{t-1} + b_t      (forward-time estimators)
 * solved per environment as an associative scan over (a, b) pairs with the
 * composition (aL, bL) o (aE, bE) = (aL*aE, aL*bE + bL) (E applied first),
 * the coefficients (a_t, b_t) being built on chip from the estimator's inputs
 * inside the scan kernel ("rl-triton: High-Performance Triton GPU Kernels for
 * Reinforcement Learning Credit Assignment", arXiv 2608.17641, abstract).
 * The seven entry points are the seven kernels of the rl-triton README,
 * section "Kernels" (one row each).
 *
 * Common conventions
 * ------------------
 * Layout      All per-step tensors are dense row-major [N, T] (element (n, t)
 *             at n*T + t); Retrace's action-valued tensors are [N, T, A]
 *             (element (n, t, a) at (n*T + t)*A + a).  N is the number of
 *             environments, T the rollout length (README, section "Usage":
 *             [num_envs, seq_len] tensors).
 * Memory      Every pointer is a DEVICE pointer on the current HIP device,
 *             allocated and owned by the caller.  The library never frees or
 *             retains caller pointers.  Outputs must not alias inputs.
 *             16-byte aligned pointers take the vectorised path (one-byte
 *             flag tensors: 4-byte aligned); any other alignment is accepted
 *             and takes a scalar-load path.
 * Flags       terminated / truncated / dones are float32 tensors (README,
 *             section "Usage", passes terminateds as a float tensor), or
 *             uint8 tensors for the *_u8 entry points; a flag is set iff its
 *             value != 0.
 * Episodes    Reverse estimators (GAE, TD(lambda), discounted returns,
 *             V-trace, Retrace): step t is a chain cut if terminated, or
 *             truncated, or t = T-1.  Terminated means the successor value is
 *             0; truncated means it is bootstrap_values[n, t]; the end of the
 *             row means it is bootstrap_value[n] (0 if that pointer is NULL).
 *             When both flags are set, terminated wins.  (README, section
 *             "Performance": GAE, V-trace, TD(lambda) and discounted returns
 *             take terminations, time-limit truncations and bootstrap values;
 *             Retrace takes both flags, mandatory and distinct, with its
 *             continuation value inside the next-state Q tensor; traces and
 *             prefix sum take a single done flag and no bootstrap.)
 *             Forward estimators: the flag at step t drops the carry from
 *             step t-1; every row starts from 0.
 * Parameters  gamma, lambda in [0, 1] and finite; rho_bar, c_bar, rho_bar_pg
 *             > 0 (+inf allowed, NaN rejected).
 * Streams     Work is enqueued on `stream` (NULL = the device's null stream),
 *             which must belong to the current HIP device (the library's
 *             own scratch is taken on the current device), and the call
 *             returns without synchronising.  Results are valid
 *             once the stream has completed.  Faults inside kernels surface at
 *             the caller's next synchronisation, as for any HIP kernel.
 * Empty       N == 0 or T == 0 is a successful no-op (pointers may be NULL).
 * Errors      A negative rlscan_status is returned, and nothing is enqueued,
 *             for: a NULL required pointer, a negative size or an element
 *             count above 2^48, a parameter out of range, an output pointer
 *             equal to an input pointer (or to the other output).  A failed
 *             HIP call (launch, allocation of the library's own scratch)
 *             returns RLSCAN_ERR_HIP / RLSCAN_ERR_ALLOC.  No C++ exception
 *             crosses this interface.
 * Scratch     Sequences that span several workgroups (long rows, or rows that
 *             do not tile evenly) use a small library-owned status buffer per
 *             (device, stream) for the single-pass decoupled look-back,
 *             allocated on first need and grown when a call needs more; it is
 *             released by rlscan_release_scratch().  Calls that use it from
 *             several host threads on one stream are serialised internally.
 *             Look-back launches of one device are also ordered across
 *             streams: such a launch on a stream other than the previous
 *             one's waits (on the GPU, through an event) for the previous
 *             look-back launch, so two of them never run at once and hold
 *             slots the other's tiles need.  The event is recorded only once
 *             look-back launches have come from more than one stream of the
 *             device (a stream used for them must then stay alive while
 *             later calls are enqueued).  Packed launches are not ordered.
 *             The scratch of a stream handle stays until
 *             rlscan_release_scratch() and is reused by a later stream that
 *             gets the same handle: destroy a stream only after its rlscan
 *             work has completed.
 * Rounding    float32 results of a call that uses the look-back (see
 *             rlscan_plan) can differ in the last bits between two runs on
 *             the same inputs: a tile composes whichever of its
 *             predecessors' published values are ready, in an order that
 *             depends on timing.  Packed calls and the int64 prefix sum are
 *             deterministic.
 * Graphs      Calls whose tiles hold whole rows (the packed mapping, see
 *             rlscan_plan: all rows in one tile, or whole rows filling at
 *             least 3/4 of a tile -- every T that divides the tile, and
 *             most other rollout lengths up to it, e.g. 20, 96, 100, 200
 *             or 1000) launch one kernel and nothing else, and may be
 *             captured into a HIP graph.  A call that needs the
 *             look-back (rlscan_plan: RLSCAN_MAP_LOOKBACK) returns
 *             RLSCAN_ERR_CAPTURE on a capturing stream: a replay would
 *             reuse the call's tag and scratch (rlscan_gae_noalloc, whose
 *             scratch never moves, is the exception; see there).
 * Thread      All entry points may be called concurrently from several host
 * safety      threads.
 */
#ifndef RLSCAN_H_
#define RLSCAN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RLSCAN_OK = 0,
    RLSCAN_ERR_NULL = -1,  /* a required pointer is NULL                        */
    RLSCAN_ERR_SHAPE = -2, /* negative N/T, A < 1, or too many elements         */
    RLSCAN_ERR_PARAM = -3, /* gamma/lambda/rho_bar/c_bar out of range           */
    RLSCAN_ERR_ALIAS = -4, /* an output pointer equals an input or other output */
    RLSCAN_ERR_HIP = -5,   /* a HIP runtime call or kernel launch failed        */
    RLSCAN_ERR_ALLOC = -6, /* the library could not allocate its scratch        */
    RLSCAN_ERR_CAPTURE = -7, /* a look-back launch on a stream under graph capture
                               (rlscan_gae_noalloc: one that would need tickets) */
    RLSCAN_ERR_SCRATCH = -8  /* rlscan_gae_noalloc: more look-back tiles than its
                                fixed array holds                                */
} rlscan_status;

/* GAE (README, Kernels table, compute_gae: a backward scan that adds each
 * step's TD error to gamma*lambda times the next advantage; Schulman et al.
 * 2016).
 *   delta_t = r_t + gamma*Vhat_{t+1} - V_t
 *   A_t     = delta_t + (cut_t ? 0 : gamma*lambda*A_{t+1})
 * in:  rewards, values, terminated [N,T]; bootstrap_value [N] or NULL (-> 0);
 *      truncated [N,T] or NULL (no truncation); bootstrap_values [N,T],
 *      required iff truncated != NULL.
 * out: advantages [N,T]. */
int rlscan_gae(const float* rewards, const float* values, const float* bootstrap_value,
               const float* terminated, const float* truncated,
               const float* bootstrap_values, float* advantages,
               int64_t N, int64_t T, float gamma, float lambda, hipStream_t stream);

/* TD(lambda) returns (README, Kernels table, compute_lambda_returns: lambda
 * returns mixing one-step TD targets with Monte-Carlo returns).
 *   G_t = r_t + gamma*Vhat_{t+1}                                 if cut_t
 *   G_t = r_t + gamma*((1-lambda)*V_{t+1} + lambda*G_{t+1})      otherwise
 * Inputs as rlscan_gae.  out: returns [N,T]. */
int rlscan_lambda_returns(const float* rewards, const float* values,
                          const float* bootstrap_value, const float* terminated,
                          const float* truncated, const float* bootstrap_values,
                          float* returns, int64_t N, int64_t T, float gamma, float lambda,
                          hipStream_t stream);

/* Discounted returns (README, Kernels table, compute_discounted_returns:
 * discounted reward-to-go).
 *   G_t = r_t + gamma*(cut_t ? Vhat_{t+1} : G_{t+1})
 * in:  rewards, terminated [N,T]; bootstrap_value [N] or NULL (pure
 *      reward-to-go at the row end); truncated [N,T] or NULL;
 *      bootstrap_values [N,T], required iff truncated != NULL.
 * out: returns [N,T]. */
int rlscan_discounted_returns(const float* rewards, const float* bootstrap_value,
                              const float* terminated, const float* truncated,
                              const float* bootstrap_values, float* returns,
                              int64_t N, int64_t T, float gamma, hipStream_t stream);

/* V-trace (README, Kernels table, compute_vtrace: importance-weighted
 * targets and advantages; Espeholt et al. 2018, IMPALA).
 *   rho_t = min(rho_bar, exp(log_rhos_t)),  c_t = min(c_bar, exp(log_rhos_t))
 *   delta_t = rho_t*(r_t + gamma*Vhat_{t+1} - V_t)
 *   vs_t  = V_t + u_t,  u_t = delta_t + (cut_t ? 0 : gamma*c_t*u_{t+1})
 *   pg_t  = rho_t*(r_t + gamma*(cut_t ? Vhat_{t+1} : vs_{t+1}) - V_t)
 * in:  rewards, values, log_rhos (log pi - log mu of the taken action),
 *      terminated [N,T]; bootstrap_value, truncated, bootstrap_values as
 *      rlscan_gae.
 * out: vs [N,T] (targets), pg_advantages [N,T].
 * Precision: with gamma*c_bar > 1 (for rlscan_vtrace_ex: gamma*lambda*c_bar
 * > 1; c_bar = +inf included) a trace coefficient gamma*c_t can exceed 1,
 * and the recurrence expands: the products of the coefficients along an
 * episode grow, and so does the weight of every rounding made before them
 * (over episodes of about 100 steps, one float32 rounding of a coefficient
 * can move a result by 1e-4 of its size).  Such calls run a float64 form of
 * the kernels -- ratio (exp), clips, TD error, scan state and epilogue in
 * float64, only vs and pg rounded to float32 -- and stay within
 * 1e-4*(1 + |exact|) of the exact result for the given float32 inputs,
 * like every other call.  That form runs at most two rounds per tile (see
 * rlscan_plan, which reports the float32 form's plan) and takes two
 * look-back status entries per tile.  A chunked rollout (the *_carry calls)
 * hands vs across chunk edges in float32: expanding traces amplify that
 * rounding too, so chunked and whole-rollout results then agree only up to
 * it. */
int rlscan_vtrace(const float* rewards, const float* values, const float* bootstrap_value,
                  const float* log_rhos, const float* terminated, const float* truncated,
                  const float* bootstrap_values, float* vs, float* pg_advantages,
                  int64_t N, int64_t T, float gamma, float rho_bar, float c_bar,
                  hipStream_t stream);

/* Retrace(lambda) (README, Kernels table, compute_retrace: off-policy return
 * with truncated importance ratios; README, section "Performance": both
 * flags mandatory, continuation value folded into next_q_values_all at every
 * step; Munos et al. 2016).
 *   EQ_t = sum_a next_target_probs[t,a]*next_q_values_all[t,a]
 *   G_t  = r_t                                         if terminated_t
 *   G_t  = r_t + gamma*EQ_t                            if truncated_t or t = T-1
 *   G_t  = r_t + gamma*(EQ_t + c'_t*(G_{t+1} - next_q_values_all[t, a_{t+1}]))
 *   c'_t = lambda*min(1, next_target_probs[t, a_{t+1}] / behaviour_probs[t+1])
 * in:  rewards [N,T]; next_q_values_all, next_target_probs [N,T,A] (Q and pi
 *      at the successor state of step t); actions [N,T] int32 (a_t);
 *      behaviour_probs [N,T] (mu(a_t | x_t)); terminated, truncated [N,T],
 *      both required.
 * out: targets [N,T].
 * Preconditions (not checked on the device): actions in [0, A) -- an
 * out-of-range action is clamped into range and gives unspecified values,
 * never an out-of-bounds access; behaviour_probs > 0. */
int rlscan_retrace(const float* rewards, const float* next_q_values_all,
                   const float* next_target_probs, const int32_t* actions,
                   const float* behaviour_probs, const float* terminated,
                   const float* truncated, float* targets,
                   int64_t N, int64_t T, int64_t A, float gamma, float lambda,
                   hipStream_t stream);

/* Eligibility traces (README, Kernels table, compute_eligibility_traces:
 * accumulating forward traces, each step adding x_t to gamma*lambda*(1-d)
 * times the previous trace).
 *   e_t = x_t + (d_t ? 0 : gamma*lambda*e_{t-1}),  e_{-1} = 0
 * in:  x, dones [N,T].  out: traces [N,T]. */
int rlscan_eligibility_traces(const float* x, const float* dones, float* traces,
                              int64_t N, int64_t T, float gamma, float lambda,
                              hipStream_t stream);

/* Episodic prefix sum (README, Kernels table, compute_episodic_prefix_sum:
 * cumulative sum restarted by the done mask), exact integer arithmetic.
 *   y_t = x_t + (d_t ? 0 : y_{t-1}),  y_{-1} = 0
 * in:  x [N,T] int32, dones [N,T] float.  out: y [N,T] int64. */
int rlscan_episodic_prefix_sum(const int32_t* x, const float* dones, int64_t* out,
                               int64_t N, int64_t T, hipStream_t stream);

/* ---- streaming one rollout through several calls (carry) -----------------
 * The rl-triton README, Kernels table, last column, serves long sequences
 * by a chunked fallback: a rollout is processed in pieces.  Each *_carry
 * entry point is the call above plus two per-row arrays:
 *   carry_in [N] or NULL  the estimator's output just past this chunk: at
 *                         t = T for the reverse estimators (GAE, TD(lambda),
 *                         discounted returns, V-trace, Retrace -- the first
 *                         step of the chunk that follows, which is therefore
 *                         processed first), at t = -1 for the forward ones
 *                         (traces, prefix sum -- the last step of the chunk
 *                         before).  V-trace takes vs_T.
 *                         With carry_in, the chunk's edge step (t = T-1,
 *                         resp. t = 0) is not an episode end: it continues
 *                         into the carry unless it is terminated, truncated
 *                         or done.  V at t = T is bootstrap_value[n] (NULL:
 *                         0).  NULL carry_in: each row is a whole rollout,
 *                         exactly as the plain call.
 *   carry_out [N] or NULL the output at the opposite edge (t = 0 reverse,
 *                         t = T-1 forward; V-trace: vs), i.e. the carry_in of
 *                         the call for the neighbouring chunk.
 * Retrace with carry_in also needs next_actions [N] (a_T, int32) and
 * next_behaviour_probs [N] (mu(a_T | x_T)) of the chunk that follows
 * (RLSCAN_ERR_NULL if missing).  Layout, ownership, streams and errors are as
 * for the plain calls; carry_out must not alias any other argument.  Calls
 * with carry arguments run kernels built for them (four or eight waves per
 * workgroup); the plain calls are unaffected. */
int rlscan_gae_carry(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* advantages,
                     float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                     hipStream_t stream);
int rlscan_lambda_returns_carry(const float* rewards, const float* values,
                                const float* bootstrap_value, const float* terminated,
                                const float* truncated, const float* bootstrap_values,
                                const float* carry_in, float* returns, float* carry_out,
                                int64_t N, int64_t T, float gamma, float lambda,
                                hipStream_t stream);
int rlscan_discounted_returns_carry(const float* rewards, const float* bootstrap_value,
                                    const float* terminated, const float* truncated,
                                    const float* bootstrap_values, const float* carry_in,
                                    float* returns, float* carry_out, int64_t N, int64_t T,
                                    float gamma, hipStream_t stream);
int rlscan_vtrace_carry(const float* rewards, const float* values, const float* bootstrap_value,
                        const float* log_rhos, const float* terminated, const float* truncated,
                        const float* bootstrap_values, const float* carry_in, float* vs,
                        float* pg_advantages, float* carry_out, int64_t N, int64_t T,
                        float gamma, float rho_bar, float c_bar, hipStream_t stream);
int rlscan_retrace_carry(const float* rewards, const float* next_q_values_all,
                         const float* next_target_probs, const int32_t* actions,
                         const float* behaviour_probs, const float* terminated,
                         const float* truncated, const float* carry_in,
                         const int32_t* next_actions, const float* next_behaviour_probs,
                         float* targets, float* carry_out, int64_t N, int64_t T, int64_t A,
                         float gamma, float lambda, hipStream_t stream);
int rlscan_eligibility_traces_carry(const float* x, const float* dones, const float* carry_in,
                                    float* traces, float* carry_out, int64_t N, int64_t T,
                                    float gamma, float lambda, hipStream_t stream);
int rlscan_episodic_prefix_sum_carry(const int32_t* x, const float* dones,
                                     const int64_t* carry_in, int64_t* out,
                                     int64_t* carry_out, int64_t N, int64_t T,
                                     hipStream_t stream);

/* ---- V-trace options ------------------------------------------------------
 * IMPALA (Espeholt et al. 2018) lets the trace coefficients carry a factor
 * lambda in [0, 1], and implementations commonly truncate the weight of the
 * policy-gradient advantage at a level rho_bar_pg of its own:
 *   c_t  = lambda*min(c_bar, exp(log_rhos_t))
 *   pg_t = min(rho_bar_pg, exp(log_rhos_t))
 *          * (r_t + gamma*(cut_t ? Vhat_{t+1} : vs_{t+1}) - V_t)
 * with rho_t, delta_t and vs_t as in rlscan_vtrace.  Every other argument is
 * as for rlscan_vtrace_carry, which is this call with lambda = 1 and
 * rho_bar_pg = rho_bar (bit for bit). */
int rlscan_vtrace_ex(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* log_rhos, const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* vs,
                     float* pg_advantages, float* carry_out, int64_t N, int64_t T, float gamma,
                     float lambda, float rho_bar, float c_bar, float rho_bar_pg,
                     hipStream_t stream);

/* ---- float-valued episodic prefix sum -------------------------------------
 * The episodic prefix sum (README, Kernels table,
 * compute_episodic_prefix_sum) of float32 values:
 *   y_t = x_t + (d_t ? 0 : y_{t-1}),  y_{-1} = carry_in[n] (NULL: 0)
 * in float32 arithmetic, summed in the scan's order (not the sequential one).
 * in:  x, dones [N,T] float32; carry_in [N] or NULL.
 * out: y [N,T] float32; carry_out [N] or NULL (y at t = T-1).
 * It is the eligibility-trace recurrence with gamma*lambda = 1. */
int rlscan_episodic_prefix_sum_f32(const float* x, const float* dones, const float* carry_in,
                                   float* out, float* carry_out, int64_t N, int64_t T,
                                   hipStream_t stream);

/* ---- one-byte flags --------------------------------------------------------
 * Each *_u8 entry point is its estimator's most general call above (the
 * *_carry call; for V-trace rlscan_vtrace_ex) with terminated, truncated or
 * dones given as uint8 [N,T]: set iff != 0, so a bool tensor qualifies as
 * is.  A flag then moves 1 byte per step instead of 4 (GAE without
 * truncation reads 9 bytes per step instead of 12).  The arithmetic is that
 * of the float-flag call with every set flag read as 1, so the results are
 * identical.  Flag tensors 4-byte aligned (and the others 16-byte aligned)
 * take the vectorised path. */
int rlscan_gae_u8(const float* rewards, const float* values, const float* bootstrap_value,
                  const uint8_t* terminated, const uint8_t* truncated,
                  const float* bootstrap_values, const float* carry_in, float* advantages,
                  float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                  hipStream_t stream);
int rlscan_lambda_returns_u8(const float* rewards, const float* values,
                             const float* bootstrap_value, const uint8_t* terminated,
                             const uint8_t* truncated, const float* bootstrap_values,
                             const float* carry_in, float* returns, float* carry_out, int64_t N,
                             int64_t T, float gamma, float lambda, hipStream_t stream);
int rlscan_discounted_returns_u8(const float* rewards, const float* bootstrap_value,
                                 const uint8_t* terminated, const uint8_t* truncated,
                                 const float* bootstrap_values, const float* carry_in,
                                 float* returns, float* carry_out, int64_t N, int64_t T,
                                 float gamma, hipStream_t stream);
int rlscan_vtrace_u8(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* log_rhos, const uint8_t* terminated, const uint8_t* truncated,
                     const float* bootstrap_values, const float* carry_in, float* vs,
                     float* pg_advantages, float* carry_out, int64_t N, int64_t T, float gamma,
                     float lambda, float rho_bar, float c_bar, float rho_bar_pg,
                     hipStream_t stream);
int rlscan_retrace_u8(const float* rewards, const float* next_q_values_all,
                      const float* next_target_probs, const int32_t* actions,
                      const float* behaviour_probs, const uint8_t* terminated,
                      const uint8_t* truncated, const float* carry_in,
                      const int32_t* next_actions, const float* next_behaviour_probs,
                      float* targets, float* carry_out, int64_t N, int64_t T, int64_t A,
                      float gamma, float lambda, hipStream_t stream);
int rlscan_eligibility_traces_u8(const float* x, const uint8_t* dones, const float* carry_in,
                                 float* traces, float* carry_out, int64_t N, int64_t T,
                                 float gamma, float lambda, hipStream_t stream);
int rlscan_episodic_prefix_sum_u8(const int32_t* x, const uint8_t* dones,
                                  const int64_t* carry_in, int64_t* out, int64_t* carry_out,
                                  int64_t N, int64_t T, hipStream_t stream);

/* ---- GAE without allocation ------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * rlscan_gae_noalloc is rlscan_gae_carry (same arguments, same results) but
 * never allocates: it calls no hipMalloc, hipFree or allocating library
 * routine and creates no event.  The look-back scratch it needs for rows
 * that span several workgroups is one fixed library array of 2 MiB + 256 B
 * per GPU (65536 tiles of 32 bytes plus two counters), held by every GPU
 * the library runs on until the process ends.
 *   Limit    A call whose plan (rlscan_plan) is RLSCAN_MAP_LOOKBACK with more
 *            than 65536 tiles (beyond 2^28 elements at 4096-element tiles)
 *            returns RLSCAN_ERR_SCRATCH, before any HIP call, with nothing
 *            enqueued.  Packed calls use no scratch and have no such limit.
 *   Sharing  Every call on one GPU uses that GPU's array, which keeps the
 *            last call's contents (the status words are tagged per call, so
 *            none needs clearing between calls).  Calls that overlap on one
 *            GPU race on it: issue them on one stream, and do not let them
 *            overlap with the library's other look-back launches on that GPU
 *            (unlike those, they are not ordered across streams).
 *   Graphs   Every call may be captured into a HIP graph.  A captured
 *            look-back call records a clear of its status words before its
 *            scan and takes a call tag reserved for captured calls (eager
 *            calls never use it), so each replay starts from cleared words
 *            and reads no other call's.  Replays share the array as calls
 *            do: keep them from overlapping each other and other look-back
 *            work of the GPU.  (Under a launch override that makes
 *            workgroups loop over tiles, a capturing stream gets
 *            RLSCAN_ERR_CAPTURE: tickets cannot be replayed.) */
int rlscan_gae_noalloc(const float* rewards, const float* values, const float* bootstrap_value,
                       const float* terminated, const float* truncated,
                       const float* bootstrap_values, const float* carry_in, float* advantages,
                       float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                       hipStream_t stream);

/* ---- several calls in one launch -------------------------------------------
 * A call of a few million elements (4096 x 128: 6-38 MB) is bound by its
 * launch and one memory round trip, not by bandwidth; a step of several such
 * calls on one stream pays that once per call.  rlscan_group runs `count`
 * independent calls in one kernel launch (up to 8 calls per launch; more are
 * split into several launches, in order): every call computes exactly what
 * its own entry point computes, with its own tiles running side by side with
 * the others'.
 *
 * Each call is described by an rlscan_call: `in` holds its inputs and `out`
 * its outputs, in the order of the estimator's plain entry point above
 * (GAE: rewards, values, bootstrap_value, terminated, truncated,
 * bootstrap_values -> advantages; V-trace: ... -> vs, pg_advantages;
 * Retrace: rewards, next_q_values_all, next_target_probs, actions,
 * behaviour_probs, terminated, truncated -> targets; traces and prefix sum:
 * x, dones -> out).  Unused entries are NULL.  V-trace reads lambda as its
 * trace factor and rho_bar_pg as its policy-gradient clip (the plain form:
 * lambda = 1, rho_bar_pg = rho_bar); the other estimators ignore rho_bar,
 * c_bar and rho_bar_pg.  With RLSCAN_CALL_BYTE_FLAGS the flags are uint8
 * (as for the *_u8 entry points).
 *
 * Every call must be one that runs as a single packed launch (rlscan_plan:
 * RLSCAN_MAP_PACKED) whose rows fit whole in the group's tile of 512 or
 * 1024 elements (T <= 1024, or N*T <= 1024), every pointer 16-byte aligned
 * (one-byte flags: 4-byte aligned), and, for Retrace, A in {4, 6, 8}.  The calls must be independent: no call may
 * write a buffer another call of the group reads or writes.
 *
 * Each call's tiles run as one contiguous stretch of the launch's workgroups,
 * in the order given (or dealt in turn with RLSCAN_FLAG_GROUP_INTERLEAVED,
 * see rlscan_set_launch_override).  The order changes the time, not the
 * results: a call that moves many bytes per tile (Retrace) is best placed
 * early, since placed last its tiles form the launch's tail.
 *
 * Returns the first failing call's status (its argument checks are those of
 * its entry point), RLSCAN_ERR_PARAM if a call cannot be grouped or names an
 * unknown estimator, RLSCAN_ERR_ALIAS for calls that are not independent;
 * nothing is enqueued then.  Streams, graphs and errors otherwise as for the
 * single calls (a grouped launch may be captured). */
enum { RLSCAN_CALL_BYTE_FLAGS = 1 };

typedef struct rlscan_call {
    int32_t estimator;       /* RLSCAN_EST_*                                   */
    int32_t flags;           /* RLSCAN_CALL_* bits                             */
    int64_t N, T;            /* rows, steps per row                            */
    int64_t A;               /* Retrace: actions per step; otherwise ignored   */
    float gamma, lambda;
    float rho_bar, c_bar, rho_bar_pg;  /* V-trace                             */
    float reserved;          /* set to 0                                       */
    const void* in[8];
    void* out[2];
} rlscan_call;

int rlscan_group(const rlscan_call* calls, int32_t count, hipStream_t stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* rlscan_status_string(int status);

/* Library version string (static storage). */
const char* rlscan_version(void);

/* Frees the look-back scratch of every (device, stream) pair; a later call
 * that needs scratch allocates it again.  The caller must make sure no
 * rlscan work is still running on any stream.  (The fixed array of
 * rlscan_gae_noalloc is not affected.) */
int rlscan_release_scratch(void);

/* ---- launch planning (host only; no GPU work) ---------------------------
 * The library maps the flattened N*T elements onto tiles of
 * 256*waves*rounds consecutive elements, one workgroup of 64*waves threads
 * (waves = 1, 2, 4 or 8 wave64s; 1 and 2 with one round only) per tile.
 * mapping RLSCAN_MAP_PACKED: every tile holds whole rows, no inter-workgroup
 * traffic.  A tile holds floor(tile_elems / T) rows (fewer, if needed, to
 * make their element count a multiple of 4: for odd T a multiple of 4
 * rows), or all rows when they fit; where those rows do not fill the tile,
 * its remaining lanes idle.  Chosen when the rows fill at least 3/4 of the
 * tile (T = 100: 5 rows of a 512-element tile), so rollout lengths that
 * divide no tile size pack too.  One round of work per lane (at most 2^20
 * elements) allows tiles of up to 2048 elements (Retrace: 1024), so for
 * example T = 702 (two rows, 69 % of 2048) or odd T = 171 (eight rows,
 * 67 %) take the look-back.
 * mapping RLSCAN_MAP_LOOKBACK: rows span tiles; carries travel between
 * workgroups through the single-pass decoupled look-back (rows longer than
 * the largest tile, or rows that would fill less than 3/4 of one). */
enum { RLSCAN_MAP_AUTO = 0, RLSCAN_MAP_PACKED = 1, RLSCAN_MAP_LOOKBACK = 2 };

enum {
    RLSCAN_EST_GAE = 0, RLSCAN_EST_LAMBDA_RETURNS = 1, RLSCAN_EST_DISCOUNTED = 2,
    RLSCAN_EST_VTRACE = 3, RLSCAN_EST_RETRACE = 4, RLSCAN_EST_ELIGIBILITY = 5,
    RLSCAN_EST_PREFIX_SUM = 6
};

typedef struct {
    int32_t mapping;     /* RLSCAN_MAP_PACKED or RLSCAN_MAP_LOOKBACK         */
    int32_t rounds;      /* 4-element chunks per lane per tile (1, 2 or 4)   */
    int64_t tile_elems;  /* capacity of a tile = 4 * rounds * threads        */
    int64_t tiles;       /* number of tiles: ceil(N*T / tile_span) for the
                            look-back, ceil(N / rows per tile) for packed    */
    int64_t grid;        /* workgroups launched                              */
    int32_t threads;     /* threads per workgroup: 64, 128, 256 or 512       */
    int32_t tile_span;   /* elements of memory per tile: tile_elems, or for
                            the packed mapping the whole rows a tile holds
                            (a multiple of 4, at least 3/4 of tile_elems
                            unless the mapping is forced)                     */
} rlscan_plan_info;

/* Fills *info with the launch the library would make for this estimator and
 * shape under the current override (V-trace: its float32 form; a call whose
 * gamma*lambda*c_bar exceeds 1 runs at most two rounds per tile).  Returns
 * RLSCAN_ERR_SHAPE for invalid sizes, RLSCAN_ERR_PARAM for an unknown
 * estimator id. */
int rlscan_plan(int estimator, int64_t N, int64_t T, int64_t A, rlscan_plan_info* info);

enum {
    RLSCAN_FLAG_TICKETS = 1,          /* order look-back tiles by a ticket counter
                                         even with one workgroup per tile     */
    RLSCAN_FLAG_GROUP_INTERLEAVED = 2, /* rlscan_group: deal the workgroups to the
                                         calls' tiles in turn instead of one
                                         stretch of the grid per call: the
                                         time no longer depends on the calls'
                                         order.  The contiguous default is
                                         faster when the call moving the most
                                         bytes per tile is not last, slower
                                         when it is                         */
    RLSCAN_FLAG_LOOKBACK_GIVE_UP = 4  /* tests of the failure path: every
                                         look-back wait gives up after a few
                                         polls, as if no predecessor had
                                         published; see
                                         rlscan_lookback_timeouts            */
};

/* Overrides the planner for every later call in the process (tests and
 * benchmarks).  mapping: RLSCAN_MAP_AUTO/PACKED/LOOKBACK (PACKED is only
 * honoured where it is valid); rounds: 0 = automatic, else 1, 2 or 4;
 * waves: 0 = automatic, else 1, 2, 4 or 8 wave64s per workgroup (1 and 2
 * apply with one round; with more rounds 4 is used); grid_cap: 0 = no cap,
 * else at most this many workgroups, each looping over tiles; flags:
 * RLSCAN_FLAG_* bits.  Retrace runs one round of at most 4 waves; a call
 * with an input or output that is not aligned for the vector path runs one
 * round of 4 waves, and one with carry arguments 4 or 8 waves.  By default
 * look-back tiles are ordered by workgroup index, and by tickets only when
 * workgroups loop.  Returns RLSCAN_ERR_PARAM for other values. */
int rlscan_set_launch_override(int mapping, int rounds, int waves, int64_t grid_cap, int flags);

/* Overrides the order in which the workgroups of packed and grouped
 * launches take their tiles, for every later call in the process (tests and
 * benchmarks).  Workgroup b runs on XCD b % 8 of the MI355X; with run > 0
 * the tiles are cut into groups of 8*run and in each group XCD x takes the
 * x-th run of `run` consecutive tiles (a group cut short by the end of the
 * grid keeps tile = b).  run = 0: tile = b; run = -1: the library's own
 * choice (the default: runs of 16 for packed launches whose tile span is
 * not a multiple of 32 elements, where neighbouring tiles share a cache
 * line; tile = b otherwise and for grouped launches).  Look-back launches
 * always take tile = b.  Results do not depend on the order.  Returns
 * RLSCAN_ERR_PARAM for run < -1 or above 2^20. */
int rlscan_set_xcd_run(int64_t run);

/* Diagnostics: enqueues an empty kernel of `grid` workgroups of `threads`
 * threads on `stream` -- the launch-bound floor of a scan launch with that
 * grid and workgroup size (rlscan_plan gives both).  Returns
 * RLSCAN_ERR_SHAPE unless 1 <= grid < 2^23 and threads is a multiple of 64
 * from 64 to 1024. */
int rlscan_launch_floor(int64_t grid, int32_t threads, hipStream_t stream);

/* Diagnostics: enqueues a plain streaming copy of `bytes` bytes from `src`
 * to `dst` (device pointers, 16-byte aligned, not overlapping; bytes a
 * multiple of 16, at most about 2^37) with the same 16-byte non-temporal accesses the
 * scan kernels use: the achievable-bandwidth reference for a kernel that
 * reads and writes the same bytes.  Returns RLSCAN_ERR_SHAPE for a bad size,
 * RLSCAN_ERR_NULL, RLSCAN_ERR_PARAM for a misaligned pointer, and
 * RLSCAN_ERR_ALIAS for overlapping ranges. */
int rlscan_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

/* Diagnostics: enqueues a streaming kernel with a read:write mix -- the
 * achievable-bandwidth reference for a scan call that reads read_bytes and
 * writes write_bytes.  Each thread reads `reads` (1..16) 16-byte words of
 * `src`, then writes `writes` (1..4) words of `dst`, each the sum of the
 * words it read (every read is used before any write, as in a scan);
 * workgroups of 256 threads take consecutive spans of both buffers, with the
 * same non-temporal 16-byte accesses as the scans.  With reads = writes = 1
 * and equal sizes it is a copy.  A bandwidth reference is the fastest over
 * a few (reads, writes) choices of the call's read:write ratio (more words
 * per thread: more bytes in flight, fewer workgroups).  Buffers are device
 * pointers, 16-byte aligned, not overlapping; sizes multiples of 16.
 * Returns RLSCAN_ERR_SHAPE for bad sizes, RLSCAN_ERR_PARAM for counts out of
 * range or misaligned pointers, RLSCAN_ERR_NULL, RLSCAN_ERR_ALIAS. */
int rlscan_stream_mix(void* dst, int64_t write_bytes, const void* src, int64_t read_bytes,
                      int32_t reads, int32_t writes, hipStream_t stream);

/* Diagnostics: the streaming reference in a scan's own access pattern.
 * `src` holds `arrays_in` (1..16) consecutive arrays of read_bytes/arrays_in
 * bytes, `dst` `arrays_out` (1..4) arrays of write_bytes/arrays_out bytes;
 * word i of every output array becomes the sum of word i of every input
 * array (16-byte words, non-temporal accesses).  Each thread handles `words`
 * (1..4) indices, laid out as the scans lay out their chunks (each wave64 a
 * run of 64*words consecutive indices, a workgroup of 256 threads four
 * such runs); arrays_in * words is at most 16.  workgroups_per_cu (0, or
 * 2..8) caps the workgroups resident on a CU by giving each a share of the
 * CU's LDS (0: as many as registers allow): fewer waves in flight can suit
 * the DRAM better, as a scan kernel's register use does.  A scan call reads
 * each input at the index it writes, so this layout, beside
 * rlscan_stream_mix's spans, is a candidate for the call's achievable
 * bandwidth.  Buffers are device pointers, 16-byte aligned, not
 * overlapping.  Returns RLSCAN_ERR_SHAPE for sizes that are negative or do
 * not split into whole words per array, RLSCAN_ERR_PARAM for counts out of
 * range (or a cap the device's LDS cannot express) or misaligned pointers,
 * RLSCAN_ERR_NULL, RLSCAN_ERR_ALIAS. */
int rlscan_stream_mix_arrays(void* dst, int64_t write_bytes, const void* src, int64_t read_bytes,
                             int32_t arrays_in, int32_t arrays_out, int32_t words,
                             int32_t workgroups_per_cu, hipStream_t stream);

/* Diagnostics: waits in the look-back are bounded (a few seconds per
 * predecessor); a wait that reaches the bound is counted, its tile takes NaN
 * as its entering state, so every float result of the tile is NaN (the
 * prefix sum takes INT64_MIN: the tile's results up to its first reset are
 * INT64_MIN plus their partial sums, in wrapping int64 arithmetic), and the
 * kernel finishes.  This call waits for every device that has look-back
 * scratch, then stores the total count of such timeouts since the scratch
 * was allocated (rlscan_gae_noalloc's fixed arrays included).  A correct build never reports one; the tests assert that
 * (and force the path with RLSCAN_FLAG_LOOKBACK_GIVE_UP). */
int rlscan_lookback_timeouts(uint64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* RLSCAN_H_ */
