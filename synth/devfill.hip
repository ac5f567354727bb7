// Device fill of expert weights with the counter-based generator defined in
// synth/__init__.py (SplitMix64 output function, Irwin-Hall sum of four
// 16-bit lanes, one float32 multiply, bf16 / OCP E4M3FN round-to-nearest-
// even).  Input generation only: it lets multi-GB synthetic weight stacks be
// written in HBM without a host round trip; the tests check it bit for bit
// against the NumPy definition and the C host fill.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __host__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline int32_t irwin_hall(uint64_t v) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    return (int32_t)((lo & 0xFFFFu) + (lo >> 16) + (hi & 0xFFFFu) + (hi >> 16)) - 131070;
}

__device__ inline uint16_t bf16_rne(float a) {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline uint8_t e4m3fn_rne(float a) {
    uint32_t u = __float_as_uint(a);
    uint32_t sign = (u >> 31) << 7;
    uint32_t mu = u & 0x7FFFFFFFu;
    int e = (int)(mu >> 23) - 127;
    uint32_t code;
    if (e >= -6) {
        uint32_t mant = mu & 0x7FFFFFu;
        uint32_t r = mant >> 20, rem = mant & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) r++;
        if (r == 8u) { r = 0u; e++; }
        code = ((uint32_t)(e + 7) << 3) | r;
        if (code > 0x7Eu) code = 0x7Eu;
    } else {
        // |a| < 2^-6: exact scaling by 2^9, then round half to even
        code = (uint32_t)rintf(__uint_as_float(mu) * 512.0f);
    }
    return (uint8_t)(code | sign);
}

template <int KIND>   // 0 = bf16, 1 = fp8, 2 = block scales
__global__ void fill_kernel(void *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                            int64_t start, float c) {
    const int64_t total = n_exp * per_exp;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += stride) {
        const int64_t j = g / per_exp, n = g - j * per_exp;
        const uint64_t s = mix64(sid_base + ((uint64_t)j << 16));
        const uint64_t v = mix64(s + (uint64_t)(start + n + 1) * kGamma);
        if (KIND == 0) {
            static_cast<uint16_t *>(out)[g] = bf16_rne(__fmul_rn((float)irwin_hall(v), c));
        } else if (KIND == 1) {
            static_cast<uint8_t *>(out)[g] = e4m3fn_rne(__fmul_rn((float)irwin_hall(v), c));
        } else {
            const uint32_t sel = (uint32_t)((v >> 32) % 3u);
            const float m = sel == 0 ? 0.5f : (sel == 1 ? 1.0f : 2.0f);
            static_cast<float *>(out)[g] = __fmul_rn(c, m);
        }
    }
}

template <int KIND>
int launch(void *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp, int64_t start, float c,
           void *stream) {
    if (!out || n_exp < 0 || per_exp < 0 || start < 0) return -1;
    const int64_t total = n_exp * per_exp;
    if (total == 0) return 0;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_kernel<KIND>, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, out, sid_base, n_exp, per_exp, start, c);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

extern "C" {
int synth_dev_fill_bf16(void *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                        int64_t start, float c, void *stream) {
    return launch<0>(out, sid_base, n_exp, per_exp, start, c, stream);
}
int synth_dev_fill_fp8(void *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                       int64_t start, float c, void *stream) {
    return launch<1>(out, sid_base, n_exp, per_exp, start, c, stream);
}
int synth_dev_fill_scales(void *out, uint64_t sid_base, int64_t n_exp, int64_t per_exp,
                          int64_t start, float base, void *stream) {
    return launch<2>(out, sid_base, n_exp, per_exp, start, base, stream);
}
}
