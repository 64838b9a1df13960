/*
 * oracle.c -- plain, sequential, float64 CPU reference for the seven
 * credit-assignment estimators and for the first-order linear recurrence
 * they are all instances of.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, helper or
 * constant with the GPU library; it is deliberately slow and obvious, one
 * loop per estimator, each written as the estimator's own defining backward
 * (or forward) recursion, in the order and notation of its source.
 *
 * Sources (cited per function below):
 *   [abstract]  "rl-triton: High-Performance Triton GPU Kernels for
 *               Reinforcement Learning Credit Assignment" (arXiv 2608.17641),
 *               abstract: the seven estimators are one first-order linear
 *               recurrence solved by an associative scan, with terminated and
 *               truncated episodes treated separately.
 *   [README]    "rl-triton" project README, section "Kernels" (one table row
 *               per estimator), section "Usage" (tensors are
 *               [num_envs, seq_len], flags are float tensors) and section
 *               "Performance", paragraph under the H100 table (which
 *               estimators take terminated/truncated/bootstrap inputs, and
 *               that Retrace folds the continuation value into its
 *               next-state Q tensor).
 *   Standard published definitions where the pages give no formula:
 *   GAE (Schulman et al., 2016), V-trace (Espeholt et al., 2018, IMPALA),
 *   Retrace(lambda) (Munos et al., 2016), lambda-return (Sutton & Barto).
 *
 * Conventions shared by every function (readings of points the pages leave
 * open; each is listed with its reason in the design notes):
 *   - all arrays are row-major [N, T] (Retrace's two action-valued tensors
 *     are [N, T, A]); element (n, t) is at n*T + t;
 *   - a flag is set iff its float value is != 0;
 *   - parameters arrive as float and are widened to double, so the reference
 *     sees exactly the parameter value the GPU sees;
 *   - reverse estimators: a step t is a chain cut if it is terminated, or
 *     truncated, or the last step of the row (t = T-1).  The value of the
 *     next state seen from step t is
 *         0                        if terminated (terminated wins over
 *                                  truncated when both are set),
 *         bootstrap_values[n, t]   if truncated,
 *         bootstrap_value[n]       if t = T-1 (0 when that pointer is NULL),
 *         values[n, t+1]           otherwise;
 *   - forward estimators (traces, prefix sum): the flag at step t drops the
 *     carry coming from step t-1, and every row starts from 0.
 *   - streaming one rollout through several calls (the "carry" arguments;
 *     the pages' chunked fallback for long sequences, README, Kernels table,
 *     last column): carry_in[n], when given, is the estimator's output at the
 *     step just past this chunk -- t = T for the reverse estimators (the
 *     first step of the chunk that follows), t = -1 for the forward ones.
 *     The chunk's edge step (t = T-1, resp. t = 0) then continues into it
 *     instead of ending the episode; it still ends there when terminated,
 *     truncated (reverse) or done (forward).  V at t = T is
 *     bootstrap_value[n], and Retrace takes a_T and mu_T as next_actions[n]
 *     and next_behaviour_probs[n].  carry_out[n], when given, receives the
 *     output at the opposite edge (t = 0 reverse, t = T-1 forward; V-trace:
 *     vs), which is the carry_in of the call for the neighbouring chunk.
 *     NULL carry_in: every row is a whole rollout, as above.
 *
 * Build: gcc -O2 -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so -lm
 * Parity of the semantic readings themselves is unpinned by the pages (they
 * print no numeric example); the test suite pins every function to closed
 * forms, explicit-sum brute force in exact rationals, library routines and
 * cross-estimator identities.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static int is_set(const float* flags, int64_t i)
{
    return flags != NULL && flags[i] != 0.0f;
}

/* Value of the successor state of step (n, t) for the reverse estimators
 * (see the convention block above).  `values` may be NULL for estimators
 * that never read V at t+1 on a non-cut step (discounted returns). */
static double next_state_value(const float* values, const float* bootstrap_value,
                               const float* terminated, const float* truncated,
                               const float* bootstrap_values,
                               int64_t n, int64_t t, int64_t T)
{
    const int64_t i = n * T + t;
    if (is_set(terminated, i)) return 0.0;
    if (is_set(truncated, i)) return (double)bootstrap_values[i];
    if (t == T - 1) return bootstrap_value ? (double)bootstrap_value[n] : 0.0;
    return (double)values[i + 1];
}

/* `continues`: the row carries on past t = T-1 (a carry_in was given). */
static int is_cut(const float* terminated, const float* truncated,
                  int64_t i, int64_t t, int64_t T, int continues)
{
    return is_set(terminated, i) || is_set(truncated, i) || (t == T - 1 && !continues);
}

static double carry_of(const float* carry_in, int64_t n)
{
    return carry_in ? (double)carry_in[n] : 0.0;
}

/* ------------------------------------------------------------------------ *
 * The recurrence and its operator   [abstract]
 *
 * One step maps a state x to a*x + b.  Composing the step E (applied first)
 * with the step L (applied second) gives the step
 *     (aL, bL) o (aE, bE) = (aL*aE, aL*bE + bL),
 * which is associative with identity (1, 0).
 * ------------------------------------------------------------------------ */
void oracle_op_compose(double aL, double bL, double aE, double bE,
                       double* a_out, double* b_out)
{
    *a_out = aL * aE;
    *b_out = aL * bE + bL;
}

void oracle_op_compose_i64(int64_t aL, int64_t bL, int64_t aE, int64_t bE,
                           int64_t* a_out, int64_t* b_out)
{
    *a_out = aL * aE;
    *b_out = aL * bE + bL;
}

/* Plain sequential solution of x_t = a_t * x_{t+1} + b_t (reverse != 0,
 * x_T = 0) or x_t = a_t * x_{t-1} + b_t (reverse == 0, x_{-1} = 0), per row.
 * This is the recurrence's definition, used by the tests to check that each
 * estimator's coefficient table reproduces the estimator. */
void oracle_linear_recurrence(int64_t N, int64_t T, int reverse,
                              const double* a, const double* b, double* x)
{
    for (int64_t n = 0; n < N; ++n) {
        double state = 0.0;
        if (reverse) {
            for (int64_t t = T - 1; t >= 0; --t) {
                const int64_t i = n * T + t;
                state = a[i] * state + b[i];
                x[i] = state;
            }
        } else {
            for (int64_t t = 0; t < T; ++t) {
                const int64_t i = n * T + t;
                state = a[i] * state + b[i];
                x[i] = state;
            }
        }
    }
}

/* ------------------------------------------------------------------------ *
 * GAE   [README, Kernels table, compute_gae row: a backward scan in which
 * each step adds its TD error to gamma*lambda times the next advantage;
 * Usage section for the call shape; Schulman et al. 2016]
 *     delta_t = r_t + gamma * Vhat_{t+1} - V_t
 *     A_t     = delta_t + (cut_t ? 0 : gamma * lambda * A_{t+1})
 * ------------------------------------------------------------------------ */
void oracle_gae(int64_t N, int64_t T, float gamma_f, float lambda_f,
                const float* rewards, const float* values,
                const float* bootstrap_value, const float* terminated,
                const float* truncated, const float* bootstrap_values,
                const float* carry_in, double* advantages, double* carry_out)
{
    const double gamma = gamma_f, lambda = lambda_f;
    const int continues = carry_in != NULL;
    for (int64_t n = 0; n < N; ++n) {
        double next_adv = carry_of(carry_in, n);  /* A_T */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = n * T + t;
            const double v_next = next_state_value(values, bootstrap_value, terminated,
                                                   truncated, bootstrap_values, n, t, T);
            const double delta = (double)rewards[i] + gamma * v_next - (double)values[i];
            const double carry =
                is_cut(terminated, truncated, i, t, T, continues) ? 0.0 : next_adv;
            const double adv = delta + gamma * lambda * carry;
            advantages[i] = adv;
            next_adv = adv;
        }
        if (carry_out) carry_out[n] = advantages[n * T];
    }
}

/* ------------------------------------------------------------------------ *
 * TD(lambda) returns   [README, Kernels table, compute_lambda_returns row:
 * lambda-return targets that mix one-step TD and Monte Carlo; Sutton & Barto]
 *     G_t = r_t + gamma * Vhat_{t+1}                                  if cut_t
 *     G_t = r_t + gamma * ((1 - lambda) * V_{t+1} + lambda * G_{t+1}) otherwise
 * ------------------------------------------------------------------------ */
void oracle_lambda_returns(int64_t N, int64_t T, float gamma_f, float lambda_f,
                           const float* rewards, const float* values,
                           const float* bootstrap_value, const float* terminated,
                           const float* truncated, const float* bootstrap_values,
                           const float* carry_in, double* returns, double* carry_out)
{
    const double gamma = gamma_f, lambda = lambda_f;
    const int continues = carry_in != NULL;
    for (int64_t n = 0; n < N; ++n) {
        double next_ret = carry_of(carry_in, n);  /* G_T */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = n * T + t;
            const double v_next = next_state_value(values, bootstrap_value, terminated,
                                                   truncated, bootstrap_values, n, t, T);
            double g;
            if (is_cut(terminated, truncated, i, t, T, continues))
                g = (double)rewards[i] + gamma * v_next;
            else  /* here v_next is V_{t+1} (bootstrap_value[n] at t = T-1) */
                g = (double)rewards[i] + gamma * ((1.0 - lambda) * v_next + lambda * next_ret);
            returns[i] = g;
            next_ret = g;
        }
        if (carry_out) carry_out[n] = returns[n * T];
    }
}

/* ------------------------------------------------------------------------ *
 * Discounted returns   [README, Kernels table, compute_discounted_returns
 * row: discounted reward-to-go; Performance section for the truncation and
 * bootstrap inputs]
 *     G_t = r_t + gamma * (cut_t ? Vhat_{t+1} : G_{t+1})
 * where Vhat is 0 on termination, bootstrap_values[n,t] on truncation and
 * bootstrap_value[n] (or 0) at the end of the row.
 * ------------------------------------------------------------------------ */
void oracle_discounted_returns(int64_t N, int64_t T, float gamma_f,
                               const float* rewards, const float* bootstrap_value,
                               const float* terminated, const float* truncated,
                               const float* bootstrap_values, const float* carry_in,
                               double* returns, double* carry_out)
{
    const double gamma = gamma_f;
    const int continues = carry_in != NULL;
    for (int64_t n = 0; n < N; ++n) {
        double next_ret = carry_of(carry_in, n);  /* G_T */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = n * T + t;
            double follow;
            if (is_cut(terminated, truncated, i, t, T, continues))
                follow = next_state_value(NULL, bootstrap_value, terminated, truncated,
                                          bootstrap_values, n, t, T);
            else
                follow = next_ret;
            const double g = (double)rewards[i] + gamma * follow;
            returns[i] = g;
            next_ret = g;
        }
        if (carry_out) carry_out[n] = returns[n * T];
    }
}

/* ------------------------------------------------------------------------ *
 * V-trace   [README, Kernels table, compute_vtrace row: importance-weighted
 * targets and advantages; Espeholt et al. 2018, IMPALA, the recursive form
 * of the v-trace target and the policy-gradient advantage, and the same
 * paper's variant that multiplies every trace coefficient c_i by a factor
 * lambda in [0, 1]]
 *     ratio_t = exp(log_rho_t)
 *     rho_t = min(rho_bar, ratio_t),  c_t = lambda * min(c_bar, ratio_t)
 *     delta_t = rho_t * (r_t + gamma * Vhat_{t+1} - V_t)
 *     u_t  = delta_t + (cut_t ? 0 : gamma * c_t * u_{t+1}),   vs_t = V_t + u_t
 *     pg_t = min(rho_bar_pg, ratio_t)
 *            * (r_t + gamma * (cut_t ? Vhat_{t+1} : vs_{t+1}) - V_t)
 * log_rho_t is log pi(a_t|x_t) - log mu(a_t|x_t).  The plain form of the
 * paper is lambda = 1 and rho_bar_pg = rho_bar (one truncation level for
 * the target and the policy-gradient weight); a separate rho_bar_pg is the
 * option implementations commonly give the policy-gradient weight.
 * ------------------------------------------------------------------------ */
void oracle_vtrace(int64_t N, int64_t T, float gamma_f, float lambda_f, float rho_bar_f,
                   float c_bar_f, float rho_bar_pg_f, const float* rewards, const float* values,
                   const float* bootstrap_value, const float* log_rhos,
                   const float* terminated, const float* truncated,
                   const float* bootstrap_values, const float* carry_in, double* vs,
                   double* pg_advantages, double* carry_out)
{
    const double gamma = gamma_f, lambda = lambda_f, rho_bar = rho_bar_f, c_bar = c_bar_f;
    const double rho_bar_pg = rho_bar_pg_f;
    const int continues = carry_in != NULL;
    for (int64_t n = 0; n < N; ++n) {
        /* carry_in is vs_T; V_T is bootstrap_value[n] (or 0) */
        const double v_T = bootstrap_value ? (double)bootstrap_value[n] : 0.0;
        double next_vs = carry_of(carry_in, n);           /* vs_{t+1} */
        double next_u = continues ? next_vs - v_T : 0.0;  /* vs_{t+1} - V_{t+1} */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = n * T + t;
            const double ratio = exp((double)log_rhos[i]);
            const double rho = ratio < rho_bar ? ratio : rho_bar;
            const double c = lambda * (ratio < c_bar ? ratio : c_bar);
            const double rho_pg = ratio < rho_bar_pg ? ratio : rho_bar_pg;
            const double v_next = next_state_value(values, bootstrap_value, terminated,
                                                   truncated, bootstrap_values, n, t, T);
            const int cut = is_cut(terminated, truncated, i, t, T, continues);
            const double delta = rho * ((double)rewards[i] + gamma * v_next - (double)values[i]);
            const double u = delta + (cut ? 0.0 : gamma * c * next_u);
            const double vs_t = (double)values[i] + u;
            const double follow = cut ? v_next : next_vs;
            vs[i] = vs_t;
            pg_advantages[i] = rho_pg * ((double)rewards[i] + gamma * follow - (double)values[i]);
            next_u = u;
            next_vs = vs_t;
        }
        if (carry_out) carry_out[n] = vs[n * T];
    }
}

/* ------------------------------------------------------------------------ *
 * Retrace(lambda)   [README, Kernels table, compute_retrace row: off-policy
 * return estimate with truncated importance ratios; Performance section:
 * terminated and truncated are both required and distinct, and the
 * continuation value lives in the next-state Q tensor at every step;
 * Munos et al. 2016]
 *   next_q[n,t,:]  = Q(x_{t+1}, .)   (on truncation / at the row end: the
 *                                     true or bootstrap next state)
 *   next_pi[n,t,:] = pi(. | x_{t+1})
 *   actions[n,t]   = a_t,  behaviour_probs[n,t] = mu(a_t | x_t)
 *     EQ_t = sum_a next_pi[t,a] * next_q[t,a]
 *     G_t  = r_t                                           if terminated_t
 *     G_t  = r_t + gamma * EQ_t                            if truncated_t or t = T-1
 *     G_t  = r_t + gamma * (EQ_t + c'_t * (G_{t+1} - next_q[t, a_{t+1}]))   otherwise
 *     c'_t = lambda * min(1, next_pi[t, a_{t+1}] / behaviour_probs[t+1])
 * Returns 0, or -1 if an action outside [0, A) is met (nothing is written
 * past that row's start in that case).
 * ------------------------------------------------------------------------ */
int oracle_retrace(int64_t N, int64_t T, int64_t A, float gamma_f, float lambda_f,
                   const float* rewards, const float* next_q, const float* next_pi,
                   const int32_t* actions, const float* behaviour_probs,
                   const float* terminated, const float* truncated,
                   const float* carry_in, const int32_t* next_actions,
                   const float* next_behaviour_probs, double* targets, double* carry_out)
{
    const double gamma = gamma_f, lambda = lambda_f;
    const int continues = carry_in != NULL;
    for (int64_t n = 0; n < N; ++n) {
        double next_g = carry_of(carry_in, n);  /* G_T */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = n * T + t;
            const float* q = next_q + i * A;
            const float* p = next_pi + i * A;
            double eq = 0.0;
            for (int64_t a = 0; a < A; ++a) eq += (double)p[a] * (double)q[a];
            double g;
            if (is_set(terminated, i)) {
                g = (double)rewards[i];
            } else if (is_set(truncated, i) || (t == T - 1 && !continues)) {
                g = (double)rewards[i] + gamma * eq;
            } else {
                /* a_{t+1} and mu_{t+1}: the next chunk's first step at t = T-1 */
                const int32_t a_next = t == T - 1 ? next_actions[n] : actions[i + 1];
                const double mu_next = t == T - 1 ? (double)next_behaviour_probs[n]
                                                  : (double)behaviour_probs[i + 1];
                if (a_next < 0 || (int64_t)a_next >= A) return -1;
                const double ratio = (double)p[a_next] / mu_next;
                const double c = lambda * (ratio < 1.0 ? ratio : 1.0);
                g = (double)rewards[i] + gamma * (eq + c * (next_g - (double)q[a_next]));
            }
            targets[i] = g;
            next_g = g;
        }
        if (carry_out) carry_out[n] = targets[n * T];
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Eligibility traces   [README, Kernels table, compute_eligibility_traces
 * row: accumulating forward traces, each step adding x_t to gamma*lambda
 * times the previous trace unless the done flag is set]
 *     e_t = x_t + (d_t ? 0 : gamma * lambda * e_{t-1}),   e_{-1} = 0
 * ------------------------------------------------------------------------ */
void oracle_eligibility_traces(int64_t N, int64_t T, float gamma_f, float lambda_f,
                               const float* x, const float* dones, const float* carry_in,
                               double* traces, double* carry_out)
{
    const double gamma = gamma_f, lambda = lambda_f;
    for (int64_t n = 0; n < N; ++n) {
        double prev = carry_of(carry_in, n);  /* e_{-1} */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = n * T + t;
            const double e = (double)x[i] + (is_set(dones, i) ? 0.0 : gamma * lambda * prev);
            traces[i] = e;
            prev = e;
        }
        if (carry_out) carry_out[n] = traces[n * T + T - 1];
    }
}

/* ------------------------------------------------------------------------ *
 * Episodic prefix sum   [README, Kernels table,
 * compute_episodic_prefix_sum row: cumulative sum that restarts where the
 * done mask is set]; integer arithmetic only, int64 accumulator
 *     y_t = x_t + (d_t ? 0 : y_{t-1}),   y_{-1} = 0
 * ------------------------------------------------------------------------ */
void oracle_episodic_prefix_sum(int64_t N, int64_t T, const int32_t* x,
                                const float* dones, const int64_t* carry_in, int64_t* out,
                                int64_t* carry_out)
{
    for (int64_t n = 0; n < N; ++n) {
        int64_t prev = carry_in ? carry_in[n] : 0;  /* y_{-1} */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = n * T + t;
            const int64_t y = (int64_t)x[i] + (is_set(dones, i) ? 0 : prev);
            out[i] = y;
            prev = y;
        }
        if (carry_out) carry_out[n] = out[n * T + T - 1];
    }
}

/* ------------------------------------------------------------------------ *
 * Episodic prefix sum of float values   [README, Kernels table,
 * compute_episodic_prefix_sum row: cumulative sum that restarts where the
 * done mask is set], for float inputs; float64 accumulator
 *     y_t = x_t + (d_t ? 0 : y_{t-1}),   y_{-1} = 0
 * ------------------------------------------------------------------------ */
void oracle_episodic_prefix_sum_float(int64_t N, int64_t T, const float* x,
                                      const float* dones, const float* carry_in, double* out,
                                      double* carry_out)
{
    for (int64_t n = 0; n < N; ++n) {
        double prev = carry_of(carry_in, n);  /* y_{-1} */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = n * T + t;
            const double y = (double)x[i] + (is_set(dones, i) ? 0.0 : prev);
            out[i] = y;
            prev = y;
        }
        if (carry_out) carry_out[n] = out[n * T + T - 1];
    }
}
