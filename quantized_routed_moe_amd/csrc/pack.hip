// Load-time kernels: canonical -> packed weight repack, hash-table check,
// workspace initialisation.
#include <climits>

#include "common.hpp"

namespace qrmoe {

// One thread per 34-byte Q8_32 block.
__global__ __launch_bounds__(256) void pack_q8_kernel(const uint8_t *__restrict__ canon, uint8_t *__restrict__ packed,
                                                     int64_t n_mats, int64_t R, int64_t K) {
    const int64_t nb = K / 32;
    const int64_t total = n_mats * R * nb;
    const int64_t mat = q8_bytes(R, K);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / (R * nb), rem = i % (R * nb), r = rem / nb, b = rem % nb;
        const uint8_t *src = canon + i * 34;
        uint8_t *base = packed + m * mat;
        uint32_t words[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint8_t *p = src + 2 + 4 * j;
            words[j] = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(base + r * K + b * 32);
        dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
        dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
        uint16_t sc = (uint16_t)src[0] | ((uint16_t)src[1] << 8);
        reinterpret_cast<uint16_t *>(base + R * K)[r * nb + b] = sc;
    }
}

// One thread per 84-byte Q2_256 superblock.
__global__ __launch_bounds__(256) void pack_q2_kernel(const uint8_t *__restrict__ canon, uint8_t *__restrict__ packed,
                                                     int64_t n_mats, int64_t R, int64_t K) {
    const int64_t ns = K / 256;
    const int64_t total = n_mats * R * ns;
    const int64_t mat = q2_bytes(R, K);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / (R * ns), rem = i % (R * ns), r = rem / ns, sb = rem % ns;
        const uint8_t *src = canon + i * 84;
        uint8_t *base = packed + m * mat;
        const uint8_t *qs = src + 20;
        uint32_t words[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t wv = 0;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint32_t code = (qs[4 * j + s] >> (2 * c)) & 3u;  // weight 16j + 4s + c
                    wv |= code << (8 * c + 2 * s);
                }
            words[j] = wv;
        }
        uint4 *dst = reinterpret_cast<uint4 *>(base + r * (K / 4) + sb * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = make_uint4(words[4 * j], words[4 * j + 1], words[4 * j + 2], words[4 * j + 3]);
        uint8_t *smp = base + R * K / 4 + r * (K / 16) + sb * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) smp[j] = src[4 + j];
        uint8_t *ddp = base + R * K / 4 + R * K / 16 + (r * ns + sb) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) ddp[j] = src[j];
    }
}

hipError_t launch_pack(int fmt, const uint8_t *canon, uint8_t *packed, int64_t n_mats, int64_t rows, int64_t cols,
                       hipStream_t s) {
    const int64_t units = n_mats * rows * (fmt == kFmtQ8 ? cols / 32 : cols / 256);
    int64_t blocks = (units + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    if (fmt == kFmtQ8)
        pack_q8_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(canon, packed, n_mats, rows, cols);
    else
        pack_q2_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(canon, packed, n_mats, rows, cols);
    return hipGetLastError();
}

__global__ void check_table_init_kernel(int32_t *result) { *result = INT_MAX; }

// One thread per table row: entries in [0, E) and pairwise distinct.
__global__ __launch_bounds__(256) void check_table_kernel(const int32_t *__restrict__ table, int32_t vocab, int32_t k,
                                                         int32_t E, int32_t *result) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= vocab) return;
    const int32_t *p = table + row * k;
    bool bad = false;
    for (int j = 0; j < k; ++j) {
        int32_t e = p[j];
        if (e < 0 || e >= E) bad = true;
        for (int i = 0; i < j; ++i)
            if (p[i] == e) bad = true;
    }
    if (bad) atomicMin(result, (int32_t)row);
}

hipError_t launch_check_table(const int32_t *table, int32_t vocab, int32_t k, int32_t E, int32_t *result,
                              hipStream_t s) {
    check_table_init_kernel<<<1, 1, 0, s>>>(result);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    check_table_kernel<<<dim3((vocab + 255) / 256), dim3(256), 0, s>>>(table, vocab, k, E, result);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void ws_init_kernel(int32_t *ctl, int64_t n_words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (int64_t)gridDim.x * blockDim.x)
        ctl[i] = (i == kCtlMagic) ? kWsMagic : 0;
}

hipError_t launch_ws_init(int32_t *ctl, int64_t n_words, hipStream_t s) {
    int64_t blocks = (n_words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    ws_init_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(ctl, n_words);
    return hipGetLastError();
}

}  // namespace qrmoe
