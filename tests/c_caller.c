/* c_caller.c -- librlscan used from plain C11, the way a C application would
 * use it: include/rlscan.h and the HIP runtime API only (no C++, no Python,
 * no PyTorch).  Built with gcc and run by tests/test_c_caller.py.
 *
 *   c_caller checks   host-side behaviour of the boundary, no GPU needed:
 *                     the version string, status strings, rlscan_plan, and
 *                     the status codes of invalid calls (each is refused
 *                     before anything is enqueued);
 *   c_caller gpu      device buffers from hipMalloc, calls on a stream of
 *                     its own (GAE as in the rl-triton README's Usage
 *                     section, GAE with truncation on rows that need the
 *                     look-back, the episodic prefix sum on long rows, and
 *                     one rlscan_group launch holding a GAE and a prefix-sum
 *                     call), each result compared with the float64 oracle
 *                     (oracle/oracle.c, linked in) to 1e-4 * (1 + |ref|),
 *                     the integer prefix sum exactly.
 *
 * Prints "ok ..." and exits 0, or prints the first failure and exits 1.
 * The inputs come from a splitmix64 stream (seeded, synthetic). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rlscan.h"

/* the oracle's entry points (oracle/oracle.c) */
void oracle_gae(int64_t N, int64_t T, float gamma_f, float lambda_f, const float* rewards,
                const float* values, const float* bootstrap_value, const float* terminated,
                const float* truncated, const float* bootstrap_values, const float* carry_in,
                double* advantages, double* carry_out);
void oracle_episodic_prefix_sum(int64_t N, int64_t T, const int32_t* x, const float* dones,
                                const int64_t* carry_in, int64_t* out, int64_t* carry_out);

static int failures = 0;

#define EXPECT(cond, ...)                                           \
    do {                                                            \
        if (!(cond)) {                                              \
            fprintf(stderr, "FAIL line %d: ", __LINE__);            \
            fprintf(stderr, __VA_ARGS__);                           \
            fprintf(stderr, "\n");                                  \
            ++failures;                                             \
        }                                                           \
    } while (0)

#define HIP_OK(call)                                                         \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "FAIL line %d: %s: %s\n", __LINE__, #call,       \
                    hipGetErrorString(e_));                                  \
            exit(1);                                                         \
        }                                                                    \
    } while (0)

/* ------------------------------------------------------------ inputs */
static uint64_t rng_state;

static uint64_t splitmix64(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double uniform01(void) { return (double)(splitmix64() >> 11) * 0x1.0p-53; }
static float normal01(void) {
    const double u = 1.0 - uniform01(), v = uniform01();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static float* normals(int64_t n) {
    float* p = malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = normal01();
    return p;
}
static float* bernoulli(int64_t n, double prob) {
    float* p = malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = uniform01() < prob ? 1.0f : 0.0f;
    return p;
}

/* ------------------------------------------------------------ device copies */
static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}
static void* device_buffer(size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    return d;
}

static double max_scaled_error(const float* got, const double* ref, int64_t n) {
    double worst = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double e = fabs((double)got[i] - ref[i]) / (1.0 + fabs(ref[i]));
        if (!(e <= worst)) worst = e;  /* NaN counts as the worst */
    }
    return worst;
}

/* One GAE case: rlscan_gae on `stream` against oracle_gae. */
static void gae_case(const char* name, int64_t N, int64_t T, double p_term, double p_trunc,
                     hipStream_t stream) {
    const int64_t n = N * T;
    float* r = normals(n);
    float* v = normals(n);
    float* boot = normals(N);
    float* term = bernoulli(n, p_term);
    float* trunc = p_trunc > 0 ? bernoulli(n, p_trunc) : NULL;
    float* bvals = p_trunc > 0 ? normals(n) : NULL;
    const size_t fb = sizeof(float) * (size_t)n;
    float* d_r = to_device(r, fb);
    float* d_v = to_device(v, fb);
    float* d_boot = to_device(boot, sizeof(float) * (size_t)N);
    float* d_term = to_device(term, fb);
    float* d_trunc = trunc ? to_device(trunc, fb) : NULL;
    float* d_bvals = bvals ? to_device(bvals, fb) : NULL;
    float* d_adv = device_buffer(fb);

    const int rc = rlscan_gae(d_r, d_v, d_boot, d_term, d_trunc, d_bvals, d_adv, N, T, 0.99f,
                              0.95f, stream);
    EXPECT(rc == RLSCAN_OK, "%s: rlscan_gae returned %s", name, rlscan_status_string(rc));
    float* got = malloc(fb);
    HIP_OK(hipMemcpyAsync(got, d_adv, fb, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));

    double* ref = malloc(sizeof(double) * (size_t)n);
    oracle_gae(N, T, 0.99f, 0.95f, r, v, boot, term, trunc, bvals, NULL, ref, NULL);
    const double err = max_scaled_error(got, ref, n);
    EXPECT(err <= 1e-4, "%s: max |gpu - ref| / (1 + |ref|) = %g", name, err);
    printf("%s: %lld x %lld, max scaled error %.3g\n", name, (long long)N, (long long)T, err);

    HIP_OK(hipFree(d_r));
    HIP_OK(hipFree(d_v));
    HIP_OK(hipFree(d_boot));
    HIP_OK(hipFree(d_term));
    if (d_trunc) HIP_OK(hipFree(d_trunc));
    if (d_bvals) HIP_OK(hipFree(d_bvals));
    HIP_OK(hipFree(d_adv));
    free(r), free(v), free(boot), free(term), free(trunc), free(bvals), free(got), free(ref);
}

static int32_t* small_ints(int64_t n) {
    int32_t* p = malloc(sizeof(int32_t) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = (int32_t)(splitmix64() % 17) - 8;  /* U[-8, 8] */
    return p;
}

static int64_t count_mismatches(const int64_t* got, const int64_t* ref, int64_t n) {
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) bad += got[i] != ref[i];
    return bad;
}

/* The episodic prefix sum on long rows (look-back), exactly. */
static void prefix_case(int64_t N, int64_t T, hipStream_t stream) {
    const int64_t n = N * T;
    int32_t* x = small_ints(n);
    float* dones = bernoulli(n, 1e-3);
    int32_t* d_x = to_device(x, sizeof(int32_t) * (size_t)n);
    float* d_dones = to_device(dones, sizeof(float) * (size_t)n);
    int64_t* d_out = device_buffer(sizeof(int64_t) * (size_t)n);
    const int rc = rlscan_episodic_prefix_sum(d_x, d_dones, d_out, N, T, stream);
    EXPECT(rc == RLSCAN_OK, "prefix sum: %s", rlscan_status_string(rc));
    int64_t* got = malloc(sizeof(int64_t) * (size_t)n);
    HIP_OK(hipMemcpyAsync(got, d_out, sizeof(int64_t) * (size_t)n, hipMemcpyDeviceToHost,
                          stream));
    HIP_OK(hipStreamSynchronize(stream));
    int64_t* ref = malloc(sizeof(int64_t) * (size_t)n);
    oracle_episodic_prefix_sum(N, T, x, dones, NULL, ref, NULL);
    const int64_t bad = count_mismatches(got, ref, n);
    EXPECT(bad == 0, "prefix sum %lld x %lld: %lld elements differ", (long long)N,
           (long long)T, (long long)bad);
    printf("prefix sum: %lld x %lld, %lld elements differ\n", (long long)N, (long long)T,
           (long long)bad);
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_dones));
    HIP_OK(hipFree(d_out));
    free(x), free(dones), free(got), free(ref);
}

/* One rlscan_group launch with a GAE call and a prefix-sum call. */
static void group_case(hipStream_t stream) {
    const int64_t N1 = 64, T1 = 512, n1 = N1 * T1, N2 = 32, T2 = 128, n2 = N2 * T2;
    float* r = normals(n1);
    float* v = normals(n1);
    float* boot = normals(N1);
    float* term = bernoulli(n1, 0.01);
    int32_t* x = small_ints(n2);
    float* dones = bernoulli(n2, 0.01);
    const size_t fb = sizeof(float) * (size_t)n1;
    float* d_r = to_device(r, fb);
    float* d_v = to_device(v, fb);
    float* d_boot = to_device(boot, sizeof(float) * (size_t)N1);
    float* d_term = to_device(term, fb);
    float* d_adv = device_buffer(fb);
    int32_t* d_x = to_device(x, sizeof(int32_t) * (size_t)n2);
    float* d_dones = to_device(dones, sizeof(float) * (size_t)n2);
    int64_t* d_out = device_buffer(sizeof(int64_t) * (size_t)n2);

    rlscan_call calls[2];
    memset(calls, 0, sizeof(calls));
    calls[0].estimator = RLSCAN_EST_GAE;
    calls[0].N = N1;
    calls[0].T = T1;
    calls[0].A = 1;
    calls[0].gamma = 0.99f;
    calls[0].lambda = 0.95f;
    calls[0].in[0] = d_r;
    calls[0].in[1] = d_v;
    calls[0].in[2] = d_boot;
    calls[0].in[3] = d_term;
    calls[0].out[0] = d_adv;
    calls[1].estimator = RLSCAN_EST_PREFIX_SUM;
    calls[1].N = N2;
    calls[1].T = T2;
    calls[1].A = 1;
    calls[1].in[0] = d_x;
    calls[1].in[1] = d_dones;
    calls[1].out[0] = d_out;
    const int rc = rlscan_group(calls, 2, stream);
    EXPECT(rc == RLSCAN_OK, "rlscan_group: %s", rlscan_status_string(rc));

    float* adv = malloc(fb);
    int64_t* sums = malloc(sizeof(int64_t) * (size_t)n2);
    HIP_OK(hipMemcpyAsync(adv, d_adv, fb, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(sums, d_out, sizeof(int64_t) * (size_t)n2, hipMemcpyDeviceToHost,
                          stream));
    HIP_OK(hipStreamSynchronize(stream));
    double* ref_adv = malloc(sizeof(double) * (size_t)n1);
    int64_t* ref_sums = malloc(sizeof(int64_t) * (size_t)n2);
    oracle_gae(N1, T1, 0.99f, 0.95f, r, v, boot, term, NULL, NULL, NULL, ref_adv, NULL);
    oracle_episodic_prefix_sum(N2, T2, x, dones, NULL, ref_sums, NULL);
    const double err = max_scaled_error(adv, ref_adv, n1);
    const int64_t bad = count_mismatches(sums, ref_sums, n2);
    EXPECT(err <= 1e-4, "group GAE: max scaled error %g", err);
    EXPECT(bad == 0, "group prefix sum: %lld elements differ", (long long)bad);
    printf("group: GAE max scaled error %.3g, prefix sum %lld elements differ\n", err,
           (long long)bad);

    HIP_OK(hipFree(d_r));
    HIP_OK(hipFree(d_v));
    HIP_OK(hipFree(d_boot));
    HIP_OK(hipFree(d_term));
    HIP_OK(hipFree(d_adv));
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_dones));
    HIP_OK(hipFree(d_out));
    free(r), free(v), free(boot), free(term), free(x), free(dones), free(adv), free(sums);
    free(ref_adv), free(ref_sums);
}

static int run_gpu(void) {
    rng_state = 20261203u;
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    gae_case("GAE (README usage shape)", 64, 512, 0.01, 0.0, stream);
    gae_case("GAE with truncation, look-back", 5, 300001, 1e-4, 1e-4, stream);
    prefix_case(3, 700001, stream);
    group_case(stream);
    uint64_t timeouts = 1;
    EXPECT(rlscan_lookback_timeouts(&timeouts) == RLSCAN_OK && timeouts == 0,
           "look-back timeouts: %llu", (unsigned long long)timeouts);
    HIP_OK(hipStreamDestroy(stream));
    return failures;
}

/* ------------------------------------------------------------ host checks */
static int run_checks(void) {
    const char* v = rlscan_version();
    EXPECT(v != NULL && strncmp(v, "rlscan ", 7) == 0, "version string: %s", v ? v : "(null)");
    EXPECT(strcmp(rlscan_status_string(RLSCAN_OK), rlscan_status_string(RLSCAN_ERR_SHAPE)) != 0,
           "status strings");
    EXPECT(rlscan_status_string(12345) != NULL, "status string of an unknown code");

    /* refused before anything is enqueued: the pointers are never read */
    float* p = (float*)(uintptr_t)0x100000;  /* 16-byte aligned, not dereferenced */
    float* q = (float*)(uintptr_t)0x200000;
    float* o = (float*)(uintptr_t)0x300000;
    EXPECT(rlscan_gae(p, q, NULL, p, NULL, NULL, o, -1, 8, 0.99f, 0.95f, NULL) ==
               RLSCAN_ERR_SHAPE, "negative N");
    EXPECT(rlscan_gae(p, q, NULL, p, NULL, NULL, o, 4, 8, 1.5f, 0.95f, NULL) ==
               RLSCAN_ERR_PARAM, "gamma above 1");
    EXPECT(rlscan_gae(p, q, NULL, p, NULL, NULL, o, 4, 8, 0.99f, NAN, NULL) == RLSCAN_ERR_PARAM,
           "NaN lambda");
    EXPECT(rlscan_gae(NULL, q, NULL, p, NULL, NULL, o, 4, 8, 0.99f, 0.95f, NULL) ==
               RLSCAN_ERR_NULL, "NULL rewards");
    EXPECT(rlscan_gae(p, q, NULL, p, q, NULL, o, 4, 8, 0.99f, 0.95f, NULL) == RLSCAN_ERR_NULL,
           "truncated without bootstrap_values");
    EXPECT(rlscan_gae(p, q, NULL, p, NULL, NULL, q, 4, 8, 0.99f, 0.95f, NULL) ==
               RLSCAN_ERR_ALIAS, "output equal to an input");
    EXPECT(rlscan_gae(p, q, NULL, p, NULL, NULL, o, 0, 8, 0.99f, 0.95f, NULL) == RLSCAN_OK,
           "an empty call is a no-op");
    EXPECT(rlscan_episodic_prefix_sum((const int32_t*)p, q, (int64_t*)o, 4, -2, NULL) ==
               RLSCAN_ERR_SHAPE, "negative T");
    rlscan_call bad;
    memset(&bad, 0, sizeof(bad));
    bad.estimator = 99;
    bad.N = 1;
    bad.T = 1;
    EXPECT(rlscan_group(&bad, 1, NULL) == RLSCAN_ERR_PARAM, "unknown estimator in a group");

    rlscan_plan_info info;
    EXPECT(rlscan_plan(RLSCAN_EST_GAE, 4096, 128, 1, &info) == RLSCAN_OK &&
               info.mapping == RLSCAN_MAP_PACKED, "4096 x 128 plans packed");
    EXPECT(rlscan_plan(RLSCAN_EST_PREFIX_SUM, 8, 1 << 20, 1, &info) == RLSCAN_OK &&
               info.mapping == RLSCAN_MAP_LOOKBACK, "8 x 2^20 plans look-back");
    printf("%s\n", v);
    return failures;
}

int main(int argc, char** argv) {
    const char* mode = argc > 1 ? argv[1] : "";
    int rc;
    if (strcmp(mode, "checks") == 0)
        rc = run_checks();
    else if (strcmp(mode, "gpu") == 0)
        rc = run_gpu();
    else {
        fprintf(stderr, "usage: c_caller checks|gpu\n");
        return 2;
    }
    if (rc != 0) return 1;
    printf("ok %s\n", mode);
    return 0;
}
