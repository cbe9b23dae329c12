/* Host check of the division-free form of d = amax / 127 used by the
 * quantizer kernels: with R = f32(1/127) and q0 = f32(amax * R),
 * fma(fma(-q0, 127, amax), R, q0) must equal the IEEE quotient for every
 * non-negative finite f32 amax (subnormals included). Enumerates all of
 * them; prints the number of mismatches and exits non-zero on any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int main(void)
{
    const float R = 1.0f / 127.0f;
    uint64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 20)
    for (int64_t u = 0; u < 0x7f800000LL; ++u) {
        uint32_t b = (uint32_t)u, qb, rb;
        float x;
        memcpy(&x, &b, 4);
        volatile float ref = x / 127.0f;
        const float q0 = x * R;
        const float q = fmaf(fmaf(-q0, 127.0f, x), R, q0);
        const float rv = ref;
        memcpy(&qb, &q, 4);
        memcpy(&rb, &rv, 4);
        bad += qb != rb;
    }
    printf("mismatches %llu\n", (unsigned long long)bad);
    return bad != 0;
}
