/*
 * Reference oracle for the per-layer mixed-precision Adam update.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct CPU
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no source, header, table or helper with the HIP library and must
 * never be used as a fallback for it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread
 * (contraction off so every multiply and add below rounds on its own, as
 * written; no flush-to-zero, subnormals are kept).
 *
 * What it follows (pages named by title and section, no line numbers):
 *  - "Training 70B Models on Consumer Hardware (If You're Willing to Wait)"
 *    (bombadil.systems, frozen incremental training), section "The Math":
 *    the Adam moment updates m and v, bias correction by 1 - beta^t with a
 *    global step t, the update lr * m_hat / (sqrt(v_hat) + eps) with eps
 *    added outside the root, and the additive form in which the stored
 *    weight receives "+= delta" with delta the negated update.
 *  - Same page, section "The Assumption Everyone Makes": plain gradient
 *    descent W - lr*g, rewritten as W + (-lr*g).
 *  - The GPU-memory training article on the Cloudera community profile
 *    page, line item "Optimizer states": under BF16 mixed precision the
 *    optimizer keeps an FP32 master copy, updates it, and casts it back
 *    down to the 16-bit weight.
 *  - The MegaTrain summary (blog.hotdry.top), section on the memory
 *    bottleneck of the traditional paradigm: BF16 weights and gradients,
 *    FP32 moments.
 *  - The LoRA memory accounting on the Cloudera community article, its
 *    "everything else" part: adapter gradients are FP32 (4 bytes each).
 *    The _g32 entry points take FP32 gradients and are otherwise the same
 *    step.
 *
 * Readings where the pages leave a step open:
 *  - Arithmetic is FP64 evaluated from the stored FP32/BF16 values; every
 *    piece of state is rounded back to FP32 (round to nearest even) at the
 *    end of each step, because the method stores FP32 state.
 *  - Hyper-parameters arrive as FP64 decimals; 1 - beta and 1 - beta^t are
 *    taken in FP64.
 *  - t >= 1 counts the update being applied (t = 1 is the first step).
 *  - The 16-bit weight is bf16 round-to-nearest-even of the new FP32
 *    master; NaN becomes a quiet NaN that keeps sign and top payload bits.
 *  - SGD mode is the plain rewrite evaluated in FP32: delta = -(fl32(lr)*g)
 *    rounded to FP32, then master + delta rounded to FP32.  No FMA.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>
#include <unistd.h>

/* ---- BF16 <-> FP32, written from the IEEE-754 definitions -------------- */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* BF16 is the upper half of an FP32 pattern, so widening is exact. */
static double bf16_widen(uint16_t h) { return (double)f32_from_bits((uint32_t)h << 16); }

/* Round an FP32 value to the nearest BF16, ties to the even significand.
 * Dropping the low 16 bits is a truncation; adding half a BF16 ulp minus
 * one (0x7FFF) plus the parity of the kept part turns it into round to
 * nearest with ties going to the pattern whose last kept bit is 0.  A carry
 * out of the significand moves into the exponent, which gives the right
 * result also for rounding up to the next binade and for overflow to Inf.
 * NaN: keep the sign and top payload bits and set the quiet bit. */
uint16_t lso_oracle_bf16_rne(float x)
{
    uint32_t u = bits_from_f32(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void lso_oracle_bf16_rne_array(const float* x, uint16_t* out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i) out[i] = lso_oracle_bf16_rne(x[i]);
}

/* ---- one Adam step over a contiguous range ----------------------------- */

typedef struct {
    uint64_t lo, hi;
    float* master; float* m; float* v;
    const uint16_t* g;      /* BF16 gradients, or NULL when g32 is given */
    const float* g32;       /* FP32 gradients */
    uint16_t* w;
    double lr, beta1, beta2, eps, bc1, bc2;
} adam_job;

static void adam_range(const adam_job* j)
{
    const double b1 = j->beta1, b2 = j->beta2;
    const double one_minus_b1 = 1.0 - b1, one_minus_b2 = 1.0 - b2;
    for (uint64_t i = j->lo; i < j->hi; ++i) {
        double g = j->g32 ? (double)j->g32[i] : bf16_widen(j->g[i]);
        /* moments: exponential averages of g and g^2 */
        double m = b1 * (double)j->m[i] + one_minus_b1 * g;
        double v = b2 * (double)j->v[i] + one_minus_b2 * (g * g);
        /* bias correction with the global step t */
        double m_hat = m / j->bc1;
        double v_hat = v / j->bc2;
        /* delta is the negated step; eps sits outside the square root */
        double delta = -j->lr * m_hat / (sqrt(v_hat) + j->eps);
        /* additive write-back: stored weight += delta */
        double w = (double)j->master[i] + delta;
        j->m[i] = (float)m;
        j->v[i] = (float)v;
        j->master[i] = (float)w;
        if (j->w) j->w[i] = lso_oracle_bf16_rne(j->master[i]);
    }
}

static void* adam_thread(void* p) { adam_range((const adam_job*)p); return NULL; }

static int pick_threads(int nthreads, uint64_t n)
{
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if (nthreads > 256) nthreads = 256;
    /* below ~64K elements a thread costs more than it saves */
    uint64_t max_useful = n / 65536u + 1u;
    if ((uint64_t)nthreads > max_useful) nthreads = (int)max_useful;
    return nthreads;
}

/* One Adam step on n elements.  master, m, v: FP32 state, updated in
 * place.  g: BF16 gradient bits.  w: BF16 weight bits written from the new
 * master, or NULL to skip.  t >= 1.  nthreads <= 0 uses every online core.
 * Returns the number of threads used, or -1 on invalid arguments. */
static int adam_any(uint64_t n, float* master, float* m, float* v,
                    const uint16_t* g, const float* g32, uint16_t* w, uint64_t t,
                    double lr, double beta1, double beta2, double eps, int nthreads)
{
    if (t < 1 || !master || !m || !v || (!g && !g32)) return -1;
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    int nt = pick_threads(nthreads, n);
    adam_job jobs[256];
    pthread_t tid[256];
    uint64_t per = n / (uint64_t)nt, rem = n % (uint64_t)nt, lo = 0;
    for (int k = 0; k < nt; ++k) {
        uint64_t len = per + ((uint64_t)k < rem ? 1u : 0u);
        adam_job j = { lo, lo + len, master, m, v, g, g32, w, lr, beta1, beta2, eps, bc1, bc2 };
        jobs[k] = j;
        lo += len;
    }
    if (nt == 1) { adam_range(&jobs[0]); return 1; }
    int joined[256] = {0};
    for (int k = 1; k < nt; ++k) {
        if (pthread_create(&tid[k], NULL, adam_thread, &jobs[k]) == 0) joined[k] = 1;
        else adam_range(&jobs[k]);         /* no thread: do the range here */
    }
    adam_range(&jobs[0]);
    for (int k = 1; k < nt; ++k) if (joined[k]) pthread_join(tid[k], NULL);
    return nt;
}

int lso_oracle_adam(uint64_t n, float* master, float* m, float* v,
                    const uint16_t* g, uint16_t* w, uint64_t t,
                    double lr, double beta1, double beta2, double eps,
                    int nthreads)
{
    if (!g) return -1;
    return adam_any(n, master, m, v, g, NULL, w, t, lr, beta1, beta2, eps, nthreads);
}

/* The same step with FP32 gradients g (LoRA adapters keep FP32 grads). */
int lso_oracle_adam_g32(uint64_t n, float* master, float* m, float* v,
                        const float* g, uint16_t* w, uint64_t t,
                        double lr, double beta1, double beta2, double eps,
                        int nthreads)
{
    if (!g) return -1;
    return adam_any(n, master, m, v, NULL, g, w, t, lr, beta1, beta2, eps, nthreads);
}

/* ---- one plain SGD step (FP32, two roundings) -------------------------- */

/* master <- fl32(master + fl32(-(fl32(lr) * g))), the additive rewrite of
 * W - lr*g.  sub selects the subtractive spelling fl32(master - fl32(lr*g))
 * instead, so the two spellings can be compared bit for bit.  Built with
 * contraction off, so each operator below is one IEEE FP32 rounding. */
static int sgd_any(uint64_t n, float* master, const uint16_t* g, const float* g32,
                   uint16_t* w, double lr, int sub)
{
    if (!master || (!g && !g32)) return -1;
    const float lr32 = (float)lr;
    for (uint64_t i = 0; i < n; ++i) {
        float gi = g32 ? g32[i] : f32_from_bits((uint32_t)g[i] << 16);
        float prod = lr32 * gi;
        if (sub) {
            master[i] = master[i] - prod;
        } else {
            float delta = -prod;
            master[i] = master[i] + delta;
        }
        if (w) w[i] = lso_oracle_bf16_rne(master[i]);
    }
    return 1;
}

int lso_oracle_sgd(uint64_t n, float* master, const uint16_t* g, uint16_t* w,
                   double lr, int sub)
{
    if (!g) return -1;
    return sgd_any(n, master, g, NULL, w, lr, sub);
}

/* The same step with FP32 gradients. */
int lso_oracle_sgd_g32(uint64_t n, float* master, const float* g, uint16_t* w,
                       double lr, int sub)
{
    if (!g) return -1;
    return sgd_any(n, master, NULL, g, w, lr, sub);
}

/* ---- the bare additive write-back -------------------------------------- */

/* w <- fl32(w + delta) for FP32 w and delta: the page's "frozen_W += delta"
 * on its own, as in its persistence check (section "Verification"). */
int lso_oracle_accumulate_f32(uint64_t n, float* w, const float* delta)
{
    if (!w || !delta) return -1;
    for (uint64_t i = 0; i < n; ++i) w[i] = w[i] + delta[i];
    return 1;
}

/* ---- the squared L2 norm of a gradient --------------------------------- */

/* sum_i g_i^2 in FP64, in index order.  Progressive layer locking on the
 * frozen-incremental page (section "Progressive Layer Locking") locks a
 * layer once its gradient magnitude falls below a threshold; the magnitude
 * is read as the Euclidean norm, whose square this returns.  g: BF16 bit
 * patterns (g16) or FP32 values (g32); exactly one is non-NULL. */
double lso_oracle_sq_norm(uint64_t n, const uint16_t* g16, const float* g32)
{
    double s = 0.0;
    for (uint64_t i = 0; i < n; ++i) {
        double g = g32 ? (double)g32[i] : bf16_widen(g16[i]);
        s += g * g;
    }
    return s;
}

