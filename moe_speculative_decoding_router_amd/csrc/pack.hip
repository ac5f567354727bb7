// Packing of expert weights into the matrix-core tile layout that the FFN
// kernels stream.  One-time weight preparation, not part of a verify call.
//
// A tile is 1 KB: 16 rows x 32 k (bf16) or 16 rows x 64 k (fp8).  Inside a
// tile, 16-byte lane slot l (l = 0..63) holds row m = l % 16 and the k-range
// [8 g, 8 g + 8) (bf16) or [16 g, 16 g + 16) (fp8) of the tile, g = l / 16:
// exactly the A operand of v_mfma_f32_16x16x32_bf16 for lane l, so one
// 16-byte load per lane reads 1 KB of contiguous memory per wave.  Tiles are
// ordered row-tile major, K-tile minor for the gate/up matrices, so one row
// tile is one contiguous stream; there a row tile interleaves 8 gate rows
// (tile rows 0..7) with the 8 up rows of the same intermediate indices (tile
// rows 8..15), so one tile yields both halves of SwiGLU for 8 intermediate
// indices.  The down matrices are ordered in groups of 4 row tiles (64
// rows): group major, then K-tile, then the row tile inside the group, so the
// 4 row tiles that share an activation fragment are one contiguous 4 KB
// (bf16) block per K-tile.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                   long long n_slots, int R, int K, int esz, int interleave,
                                                   int half) {
    // one thread per 16-byte lane slot of the packed output
    const int KT = esz == 2 ? 32 : 64;
    const int nkt = K / KT;
    const long long per_expert = (long long)(R / 16) * nkt * 64;
    for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < n_slots; q += (long long)gridDim.x * 256) {
        const long long e = q / per_expert;
        const long long rem = q - e * per_expert;
        const int l = (int)(rem & 63);
        const long long tile = rem >> 6;
        const int m = l & 15, g = l >> 4;
        int row, kt;
        if (interleave) {
            // gate-up: row tile major, then K-tile; 8 gate rows + 8 up rows
            const int rt = (int)(tile / nkt);
            kt = (int)(tile - (long long)rt * nkt);
            row = m < 8 ? 8 * rt + m : half + 8 * rt + (m - 8);
        } else {
            // down: groups of 4 row tiles (64 rows), then K-tile, then the
            // row tile inside the group
            const int grp = (int)(tile / (4LL * nkt));
            const int rem2 = (int)(tile - (long long)grp * 4 * nkt);
            kt = rem2 >> 2;
            row = 16 * (4 * grp + (rem2 & 3)) + m;
        }
        const int k = kt * KT + g * (KT / 4);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(src + ((e * R + row) * (long long)K + k) * esz);
        *reinterpret_cast<u32x4 *>(dst + q * 16) = v;
    }
}

// ---------------------------------------------------------------------------
// Read probe: streams n16 16-byte words with the load pattern of the FFN
// kernels (each wave reads 1 KB of contiguous memory per non-temporal
// 16-byte load per lane, four loads in flight; one workgroup of 8 waves per
// compute unit) and folds them into an XOR checksum, so every byte is used.
// Its rate is the streaming ceiling the FFN kernels are measured against.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_nt16(const uint8_t *ptr) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
}

__global__ __launch_bounds__(512) void read_probe_kernel(const uint8_t *__restrict__ src, long long n16,
                                                         uint32_t *sink) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long long nw = (long long)gridDim.x * 8;
    const long long nchunks = n16 / 64;  // whole 1 KB chunks
    long long c = (long long)blockIdx.x * 8 + w;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (; c + 3 * nw < nchunks; c += 4 * nw) {
        const u32x4 a0 = ld_nt16(src + ((c)*64 + lane) * 16);
        const u32x4 a1 = ld_nt16(src + ((c + nw) * 64 + lane) * 16);
        const u32x4 a2 = ld_nt16(src + ((c + 2 * nw) * 64 + lane) * 16);
        const u32x4 a3 = ld_nt16(src + ((c + 3 * nw) * 64 + lane) * 16);
        acc ^= (a0 ^ a1) ^ (a2 ^ a3);
    }
    for (; c < nchunks; c += nw) acc ^= ld_nt16(src + (c * 64 + lane) * 16);
    if (blockIdx.x == 0 && w == 0) {  // the words past the last whole chunk
        const long long i = nchunks * 64 + lane;
        if (i < n16) acc ^= ld_nt16(src + i * 16);
    }
    unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= (unsigned)__shfl_xor((int)x, o);
    if (lane == 0) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int n_cu, hipStream_t s) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(n_cu), dim3(512), 0, s, static_cast<const uint8_t *>(src),
                       (long long)(bytes / 16), sink);
    return hipGetLastError();
}

hipError_t launch_pack(const void *src, void *dst, int E, int R, int K, int esz, int interleave, int half,
                       hipStream_t s) {
    const long long n_slots = (long long)E * (R / 16) * (K / (esz == 2 ? 32 : 64)) * 64;
    long long blocks = (n_slots + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint8_t *>(src),
                       static_cast<uint8_t *>(dst), n_slots, R, K, esz, interleave, half);
    return hipGetLastError();
}

}  // namespace moe
