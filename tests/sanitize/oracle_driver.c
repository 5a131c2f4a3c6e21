/*
 * Drives every entry point of the oracle (oracle/adam_oracle.c) on arrays of
 * exactly n elements -- n = 0, 1, ragged sizes, a size that splits unevenly
 * over threads -- with NaN, Inf, subnormal and zero values, one and several
 * threads, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any read or write past an array, use of freed memory, leak or undefined
 * operation ends the run with an error.  Exit status 0 when all calls
 * returned their documented codes.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t lso_oracle_bf16_rne(float x);
void lso_oracle_bf16_rne_array(const float* x, uint16_t* out, uint64_t n);
int lso_oracle_adam(uint64_t n, float* master, float* m, float* v, const uint16_t* g, uint16_t* w,
                    uint64_t t, double lr, double beta1, double beta2, double eps, int nthreads);
int lso_oracle_adam_g32(uint64_t n, float* master, float* m, float* v, const float* g, uint16_t* w,
                        uint64_t t, double lr, double beta1, double beta2, double eps, int nthreads);
int lso_oracle_sgd(uint64_t n, float* master, const uint16_t* g, uint16_t* w, double lr, int sub);
int lso_oracle_sgd_g32(uint64_t n, float* master, const float* g, uint16_t* w, double lr, int sub);
int lso_oracle_accumulate_f32(uint64_t n, float* w, const float* delta);
double lso_oracle_sq_norm(uint64_t n, const uint16_t* g16, const float* g32);

static uint32_t state = 12345u;
static uint32_t next_u32(void)
{
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    return state;
}

static float value(uint64_t i)
{
    static const float special[] = {0.0f, -0.0f, 1e-45f, -3e-39f, 1.0f, -2.5f};
    if (i % 97 == 3) return NAN;
    if (i % 89 == 5) return INFINITY;
    if (i % 83 == 7) return special[i % 6];
    return ((float)(next_u32() & 0xFFFFFF) / 16777216.0f - 0.5f) * 0.04f;
}

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "oracle driver: %s failed at line %d\n", #cond, __LINE__); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static void run(uint64_t n, int threads)
{
    /* exactly n elements each, so a one-element overrun is caught */
    float* master = malloc(n ? n * sizeof(float) : 1);
    float* m = calloc(n ? n : 1, sizeof(float));
    float* v = calloc(n ? n : 1, sizeof(float));
    float* g32 = malloc(n ? n * sizeof(float) : 1);
    uint16_t* g16 = malloc(n ? n * sizeof(uint16_t) : 1);
    uint16_t* w = malloc(n ? n * sizeof(uint16_t) : 1);
    float* delta = malloc(n ? n * sizeof(float) : 1);
    for (uint64_t i = 0; i < n; ++i) {
        master[i] = value(i);
        g32[i] = value(i + 1) * 1e-2f;
        delta[i] = value(i + 2);
    }
    lso_oracle_bf16_rne_array(g32, g16, n);
    for (uint64_t t = 1; t <= 3; ++t) {
        EXPECT(lso_oracle_adam(n, master, m, v, g16, w, t, 1e-3, 0.9, 0.999, 1e-8, threads) >= 1);
        EXPECT(lso_oracle_adam(n, master, m, v, g16, NULL, t, 1e-3, 0.9, 0.999, 1e-8, threads) >= 1);
        EXPECT(lso_oracle_adam_g32(n, master, m, v, g32, w, t, 1e-3, 0.9, 0.999, 1e-8, threads) >= 1);
    }
    EXPECT(lso_oracle_adam(n, master, m, v, NULL, w, 1, 1e-3, 0.9, 0.999, 1e-8, threads) == -1);
    EXPECT(lso_oracle_sgd(n, master, g16, w, 1e-2, 0) == 1);
    EXPECT(lso_oracle_sgd(n, master, g16, NULL, 1e-2, 1) == 1);
    EXPECT(lso_oracle_sgd_g32(n, master, g32, w, 1e-2, 0) == 1);
    EXPECT(lso_oracle_sgd(n, master, NULL, w, 1e-2, 0) == -1);
    EXPECT(lso_oracle_accumulate_f32(n, master, delta) == 1);
    EXPECT(lso_oracle_accumulate_f32(n, NULL, delta) == -1);
    double a = lso_oracle_sq_norm(n, g16, NULL);
    double b = lso_oracle_sq_norm(n, NULL, g32);
    EXPECT(n > 0 || (a == 0.0 && b == 0.0));
    free(master);
    free(m);
    free(v);
    free(g32);
    free(g16);
    free(w);
    free(delta);
}

int main(void)
{
    static const uint64_t sizes[] = {0, 1, 2, 3, 7, 64, 1023, 4097, 100003};
    static const int threads[] = {1, 3, 8};
    for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; ++i)
        for (size_t k = 0; k < sizeof threads / sizeof threads[0]; ++k) run(sizes[i], threads[k]);
    /* every BF16 rounding of the FP32 patterns around the special values */
    for (uint32_t u = 0x7F7F0000u; u != 0x7F810000u; ++u) {
        float x;
        memcpy(&x, &u, 4);
        (void)lso_oracle_bf16_rne(x);
    }
    if (failures) return 1;
    printf("oracle driver: all calls returned their documented codes\n");
    return 0;
}
