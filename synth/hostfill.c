/* Host (CPU) fill of expert weights with the counter-based generator that
 * synth/__init__.py defines (SplitMix64 output function, Irwin-Hall sum of
 * the four 16-bit lanes, one float32 multiply, then bf16 or OCP E4M3FN
 * round-to-nearest-even).  Input generation only: tests and the benchmark
 * use it to regenerate, on the host, exactly the weights that the device
 * fill wrote.  Built with gcc -O2 -fopenmp; no fast-math. */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline int32_t irwin_hall(uint64_t v) {
    int32_t s = (int32_t)(v & 0xFFFF) + (int32_t)((v >> 16) & 0xFFFF) +
                (int32_t)((v >> 32) & 0xFFFF) + (int32_t)(v >> 48);
    return s - 131070;
}

static inline uint16_t bf16_rne(float a) {
    uint32_t u;
    memcpy(&u, &a, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline uint8_t e4m3fn_rne(float a) {
    uint32_t u;
    memcpy(&u, &a, 4);
    uint8_t sign = (uint8_t)((u >> 31) << 7);
    float mag = fabsf(a);
    uint32_t mu;
    memcpy(&mu, &mag, 4);
    int e = (int)(mu >> 23) - 127;
    uint32_t code;
    if (e >= -6) {
        uint32_t mant = mu & 0x7FFFFFu;
        uint32_t r = mant >> 20, rem = mant & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) r++;
        if (r == 8) { r = 0; e++; }
        code = ((uint32_t)(e + 7) << 3) | r;
        if (code > 0x7Eu) code = 0x7Eu;
    } else {
        code = (uint32_t)nearbyint((double)mag * 512.0);
    }
    return (uint8_t)(code | sign);
}

void synth_host_fill_bf16(uint16_t *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                          int64_t start, float c) {
    for (int64_t j = 0; j < n_exp; ++j) {
        uint64_t s = mix64(sid_base + ((uint64_t)j << 16));
        uint16_t *o = out + j * per_exp;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < per_exp; ++n) {
            uint64_t v = mix64(s + (uint64_t)(start + n + 1) * GAMMA);
            o[n] = bf16_rne((float)irwin_hall(v) * c);
        }
    }
}

void synth_host_fill_fp8(uint8_t *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                         int64_t start, float c) {
    for (int64_t j = 0; j < n_exp; ++j) {
        uint64_t s = mix64(sid_base + ((uint64_t)j << 16));
        uint8_t *o = out + j * per_exp;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < per_exp; ++n) {
            uint64_t v = mix64(s + (uint64_t)(start + n + 1) * GAMMA);
            o[n] = e4m3fn_rne((float)irwin_hall(v) * c);
        }
    }
}

void synth_host_fill_scales(float *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                            int64_t start, float base) {
    static const float mult[3] = {0.5f, 1.0f, 2.0f};
    for (int64_t j = 0; j < n_exp; ++j) {
        uint64_t s = mix64(sid_base + ((uint64_t)j << 16));
        for (int64_t n = 0; n < per_exp; ++n) {
            uint64_t v = mix64(s + (uint64_t)(start + n + 1) * GAMMA);
            out[j * per_exp + n] = base * mult[(v >> 32) % 3u];
        }
    }
}
