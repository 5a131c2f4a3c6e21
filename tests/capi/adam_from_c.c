/* The C ABI from plain C: `steps` Adam steps over one block of n elements
 * (planar state, BF16 gradients, BF16 weight output) through lso_adam_step.
 *
 *   adam_from_c DIR N STEPS
 *
 * reads DIR/master.f32 (n floats) and DIR/grad_<t>.bf16 (n uint16, t = 1..STEPS),
 * starts from m = v = 0 with lr 1e-3, beta1 0.9, beta2 0.999, eps 1e-8, and
 * writes DIR/out_master.f32, out_m.f32, out_v.f32 and out_weight.bf16.
 * Exit status 0 on success; messages on stderr otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lso.h"

static int io(const char* dir, const char* name, void* buf, size_t bytes, int write)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, write ? "wb" : "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); return -1; }
    const size_t k = write ? fwrite(buf, 1, bytes, f) : fread(buf, 1, bytes, f);
    fclose(f);
    if (k != bytes) { fprintf(stderr, "short %s of %s\n", write ? "write" : "read", path); return -1; }
    return 0;
}

#define HIP_OK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); return 1; } } while (0)

int main(int argc, char** argv)
{
    if (argc != 4) { fprintf(stderr, "usage: %s DIR N STEPS\n", argv[0]); return 2; }
    const char* dir = argv[1];
    const size_t n = strtoull(argv[2], NULL, 10);
    const int steps = atoi(argv[3]);
    if (n == 0 || steps < 1) { fprintf(stderr, "bad arguments\n"); return 2; }
    float* host_f = malloc(4 * n);
    uint16_t* host_h = malloc(2 * n);
    if (!host_f || !host_h) return 1;
    /* one device buffer: master | m | v (4 KB aligned each) | grad | weight */
    const size_t a4 = (4 * n + 4095) & ~(size_t)4095, a2 = (2 * n + 4095) & ~(size_t)4095;
    char* dev = NULL;
    HIP_OK(hipMalloc((void**)&dev, 3 * a4 + 2 * a2));
    HIP_OK(hipMemset(dev, 0, 3 * a4 + 2 * a2));
    if (io(dir, "master.f32", host_f, 4 * n, 0)) return 1;
    HIP_OK(hipMemcpy(dev, host_f, 4 * n, hipMemcpyHostToDevice));
    lso_block b;
    memset(&b, 0, sizeof b);
    b.base = dev;
    b.n = n;
    b.off_master = 0;
    b.off_m = a4;
    b.off_v = 2 * a4;
    b.off_grad = 3 * a4;
    b.off_weight = 3 * a4 + a2;
    b.grad_dtype = LSO_DT_BF16;
    b.weight_dtype = LSO_DT_BF16;
    b.opt = LSO_OPT_ADAM;
    b.layout = LSO_LAYOUT_PLANAR;
    b.lr = 1e-3;
    b.beta1 = 0.9;
    b.beta2 = 0.999;
    b.eps = 1e-8;
    for (int t = 1; t <= steps; ++t) {
        char name[64];
        snprintf(name, sizeof name, "grad_%d.bf16", t);
        if (io(dir, name, host_h, 2 * n, 0)) return 1;
        HIP_OK(hipMemcpy(dev + b.off_grad, host_h, 2 * n, hipMemcpyHostToDevice));
        b.t = (uint64_t)t;
        const lso_status s = lso_adam_step(&b, 1, NULL);
        if (s != LSO_OK) {
            fprintf(stderr, "lso_adam_step: %s: %s\n", lso_status_string(s), lso_last_error());
            return 1;
        }
        HIP_OK(hipDeviceSynchronize());
    }
    const char* names[3] = {"out_master.f32", "out_m.f32", "out_v.f32"};
    for (int k = 0; k < 3; ++k) {
        HIP_OK(hipMemcpy(host_f, dev + k * a4, 4 * n, hipMemcpyDeviceToHost));
        if (io(dir, names[k], host_f, 4 * n, 1)) return 1;
    }
    HIP_OK(hipMemcpy(host_h, dev + b.off_weight, 2 * n, hipMemcpyDeviceToHost));
    if (io(dir, "out_weight.bf16", host_h, 2 * n, 1)) return 1;
    HIP_OK(hipFree(dev));
    free(host_f);
    free(host_h);
    return 0;
}
