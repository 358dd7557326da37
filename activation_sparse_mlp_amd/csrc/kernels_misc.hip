// Small kernels of libspffn: threshold, mask compaction, hot-first order, row
// permutation, 4-bit block split, RMS norm and the fixed-order partial-sum
// reduction.
#include "device.h"

namespace spffn {

// ---------------------------------------------------------------------------
// threshold: mask[i] = logits[i] > t  (strict; NaN compares false)
// ---------------------------------------------------------------------------
__global__ void threshold_kernel(const float *__restrict__ logits, int64_t n, float t,
                                 uint8_t *__restrict__ mask) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        mask[i] = (uint8_t)(logits[i] > t);
}

hipError_t launch_threshold(const float *logits, int64_t n, float t, uint8_t *mask,
                            hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    threshold_kernel<<<(int)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>(logits, n, t, mask);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// compaction: one workgroup of 1024 threads.  Thread t owns the contiguous byte
// range [t*per, (t+1)*per) of the mask (per a multiple of 16, read as 128-bit
// words where the range is whole and aligned), counts its set bytes, takes an
// exclusive block scan of the counts, and writes its indices in ascending
// order at its offset.  The output order is therefore ascending overall.
// ---------------------------------------------------------------------------
constexpr int kCompactThreads = 1024;

__device__ __forceinline__ int nonzero_bytes(uint32_t v) {
    v |= v >> 4;
    v |= v >> 2;
    v |= v >> 1;
    return __popc(v & 0x01010101u);
}

__device__ __forceinline__ int block_exclusive_scan(int v, int *lds_waves, int *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) lds_waves[wv] = incl;
    __syncthreads();
    if (wv == 0) {
        int w = lane < nw ? lds_waves[lane] : 0;
        int wi = w;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(wi, o, 64);
            if (lane >= o) wi += u;
        }
        if (lane < nw) lds_waves[lane] = wi - w;  // exclusive prefix of wave totals
        if (lane == nw - 1) lds_waves[64] = wi;
    }
    __syncthreads();
    *total = lds_waves[64];
    return lds_waves[wv] + incl - v;
}

// Register path: when every thread's range is at most kCompactWords 16-byte
// words, the words are loaded once (all loads in flight), counted, and the
// indices are written straight from the registers after the scan.
constexpr int kCompactWords = 4;

__device__ __forceinline__ uint4 load_mask_word(const uint8_t *__restrict__ mask, int i, int end,
                                                bool vec) {
    if (vec && i + 16 <= end) return *reinterpret_cast<const uint4 *>(mask + i);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int k = i; k < min(end, i + 16); ++k)
        w[(k - i) >> 2] |= (uint32_t)(mask[k] != 0 ? 1u : 0u) << (8 * ((k - i) & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(const uint8_t *__restrict__ mask,
                                                                  int n, int32_t *__restrict__ idx,
                                                                  int32_t *__restrict__ count,
                                                                  int32_t *__restrict__ count2) {
    __shared__ int lds[65];
    const int64_t per = (((int64_t)n + kCompactThreads - 1) / kCompactThreads + 15) & ~(int64_t)15;
    const int beg = (int)min((int64_t)n, (int64_t)threadIdx.x * per);
    const int end = (int)min((int64_t)n, (int64_t)beg + per);
    const bool vec = ((reinterpret_cast<uintptr_t>(mask) & 15) == 0);
    int total;
    if (per <= 16 * kCompactWords) {
        uint4 w[kCompactWords];
#pragma unroll
        for (int q = 0; q < kCompactWords; ++q) {
            const int i = beg + 16 * q;
            w[q] = i < end ? load_mask_word(mask, i, end, vec) : make_uint4(0, 0, 0, 0);
        }
        int c = 0;
#pragma unroll
        for (int q = 0; q < kCompactWords; ++q)
            c += nonzero_bytes(w[q].x) + nonzero_bytes(w[q].y) + nonzero_bytes(w[q].z) +
                 nonzero_bytes(w[q].w);
        int o = block_exclusive_scan(c, lds, &total);
#pragma unroll
        for (int q = 0; q < kCompactWords; ++q) {
            const uint32_t ws[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = beg + 16 * q + 4 * m + b;
                    if (i < end && ((ws[m] >> (8 * b)) & 0xFFu)) idx[o++] = i;
                }
            }
        }
    } else {
        int c = 0;
        for (int i = beg; i < end; i += 16) {
            if (vec && i + 16 <= end) {
                const uint4 w = *reinterpret_cast<const uint4 *>(mask + i);
                c += nonzero_bytes(w.x) + nonzero_bytes(w.y) + nonzero_bytes(w.z) +
                     nonzero_bytes(w.w);
            } else {
                for (int k = i; k < min(end, i + 16); ++k) c += (mask[k] != 0);
            }
        }
        int o = block_exclusive_scan(c, lds, &total);
        for (int i = beg; i < end; ++i)
            if (mask[i]) idx[o++] = i;
    }
    if (threadIdx.x == 0) {
        *count = total;
        if (count2) *count2 = total;
    }
}

hipError_t launch_compact(const uint8_t *mask, int n, int32_t *idx, int32_t *count,
                          hipStream_t s, int32_t *count2) {
    compact_kernel<<<1, kCompactThreads, 0, s>>>(mask, n, idx, count, count2);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// hot-first order: rank_i = #{j : c_j > c_i} + #{j < i : c_j == c_i};
// perm[rank_i] = i.  O(n^2) integer comparisons, load time only.  A block of
// 16 waves ranks 64 neurons (one per lane): the counts pass through LDS in
// tiles of 1024, each wave compares its lanes' neurons against 64 entries of
// every tile (an LDS broadcast per entry), and the 16 partial ranks are added
// at the end.  (One thread per neuron over the whole array left most SIMDs
// idle: 0.81 ms at 28672 neurons.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void hot_first_order_kernel(const int32_t *__restrict__ counts,
                                                               int n, int32_t *__restrict__ perm) {
    __shared__ int32_t tile[1024];
    __shared__ int32_t part[16][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int i = blockIdx.x * 64 + lane;
    const int ci = i < n ? counts[i] : 0;
    int rank = 0;
    for (int base = 0; base < n; base += 1024) {
        __syncthreads();
        tile[threadIdx.x] = base + (int)threadIdx.x < n ? counts[base + threadIdx.x] : 0;
        __syncthreads();
        const int t1 = min(wv * 64 + 64, n - base);
        for (int t = wv * 64; t < t1; ++t) {
            const int cj = tile[t];
            rank += (cj > ci) | ((cj == ci) & (base + t < i));
        }
    }
    part[wv][lane] = rank;
    __syncthreads();
    if (wv == 0 && i < n) {
        int r = 0;
        for (int w = 0; w < 16; ++w) r += part[w][lane];
        perm[r] = i;
    }
}

hipError_t launch_hot_first_order(const int32_t *counts, int n, int32_t *perm, hipStream_t s) {
    hot_first_order_kernel<<<(n + 63) / 64, 1024, 0, s>>>(counts, n, perm);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// row permutation: dst[k] = src[perm[k]], rows of row_bytes (multiple of 4)
// ---------------------------------------------------------------------------
__global__ void permute_rows_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                    const int32_t *__restrict__ perm, int rows, int64_t row_bytes) {
    const int k = blockIdx.x;
    if (k >= rows) return;
    const int from = perm[k];
    if (from < 0 || from >= rows) return;  // not a permutation entry: row left as is
    const uint8_t *s = src + (int64_t)from * row_bytes;
    uint8_t *d = dst + (int64_t)k * row_bytes;
    const bool v16 = ((row_bytes & 15) == 0) && ((reinterpret_cast<uintptr_t>(src) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(dst) & 15) == 0);
    const int64_t step = (int64_t)gridDim.y * blockDim.x;
    if (v16) {
        const int64_t nv = row_bytes / 16;
        for (int64_t t = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; t < nv; t += step)
            reinterpret_cast<uint4 *>(d)[t] = reinterpret_cast<const uint4 *>(s)[t];
    } else {
        const int64_t nw = row_bytes / 4;
        for (int64_t t = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; t < nw; t += step)
            reinterpret_cast<uint32_t *>(d)[t] = reinterpret_cast<const uint32_t *>(s)[t];
    }
}

hipError_t launch_permute_rows(const void *src, void *dst, const int32_t *perm, int rows,
                               int64_t row_bytes, hipStream_t s) {
    int64_t units = row_bytes / 16 + 1;
    int by = (int)((units + 255) / 256);
    if (by > 64) by = 64;
    dim3 grid(rows, by);
    permute_rows_kernel<<<grid, 256, 0, s>>>((const uint8_t *)src, (uint8_t *)dst, perm, rows,
                                             row_bytes);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 4-bit block split: 18-byte blocks -> [codes 16 B per block][scales 2 B per block]
// ---------------------------------------------------------------------------
__global__ void q4_0_repack_kernel(const uint8_t *__restrict__ aos, uint8_t *__restrict__ soa,
                                   int64_t nblocks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint16_t *scales = reinterpret_cast<uint16_t *>(soa + nblocks * 16);
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
        const uint8_t *src = aos + b * 18;
        // 18-byte blocks are only 2-byte aligned: read 9 halfwords
        const uint16_t *h = reinterpret_cast<const uint16_t *>(src);
        scales[b] = h[0];
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) w[m] = (uint32_t)h[1 + 2 * m] | ((uint32_t)h[2 + 2 * m] << 16);
        reinterpret_cast<uint4 *>(soa)[b] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_q4_0_repack(const void *aos, void *soa, int rows, int cols, hipStream_t s) {
    const int64_t nblocks = (int64_t)rows * (cols / 32);
    int64_t blocks = (nblocks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    q4_0_repack_kernel<<<(int)blocks, 256, 0, s>>>((const uint8_t *)aos, (uint8_t *)soa, nblocks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fill / RMS norm / fixed-order reduction
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t *p, int32_t v, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, int32_t v, int n, hipStream_t s) {
    fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, v, n);
    return hipGetLastError();
}

// dst[i] = src[i] for 4-byte words (device-to-device copy as a kernel, so a
// captured graph holds only kernel nodes)
__global__ void copy_words_kernel(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst,
                                  int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

hipError_t launch_copy_words(const void *src, void *dst, int64_t n_words, hipStream_t s) {
    int64_t blocks = (n_words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    copy_words_kernel<<<(int)blocks, 256, 0, s>>>((const uint32_t *)src, (uint32_t *)dst, n_words);
    return hipGetLastError();
}

// n_b = h_b / sqrt(mean(h_b^2) + eps), one workgroup per token.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ h, int d, float eps,
                                                      float *__restrict__ out) {
    __shared__ float red[4];
    const float *hb = h + (size_t)blockIdx.x * d;
    float *ob = out + (size_t)blockIdx.x * d;
    float ss = 0.0f;
    for (int k = threadIdx.x; k < d; k += blockDim.x) ss = fmaf(hb[k], hb[k], ss);
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float den = sqrtf(tot / (float)d + eps);
    for (int k = threadIdx.x; k < d; k += blockDim.x) ob[k] = hb[k] / den;
}

// ---------------------------------------------------------------------------
// stream read (measurement only): every 16-byte word of a buffer is read once
// with a non-temporal load, 8 loads in flight per thread, 4096 workgroups in a
// grid-stride loop; each workgroup folds its words with XOR and stores the
// result to its own sink word (no atomics: thousands of them on one address
// would serialise at the end of the launch), so no load can be dropped.  Its
// bandwidth is the read ceiling the decode kernels are compared with.
// ---------------------------------------------------------------------------
typedef unsigned int stream_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamSinkWords = SPFFN_STREAM_SINK_WORDS;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p,
                                                          int64_t n16, uint32_t *sink) {
    // sink words no workgroup owns are cleared by workgroup 0
    if (blockIdx.x == 0)
        for (int k = gridDim.x + threadIdx.x; k < kStreamSinkWords; k += blockDim.x) sink[k] = 0;
    constexpr int U = 8;
    __shared__ uint32_t red[4];
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
        stream_u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = i < n16 ? __builtin_nontemporal_load(
                                 reinterpret_cast<const stream_u32x4 *>(p + i))
                           : stream_u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    int64_t blocks = (n16 + 256 * 8 - 1) / (256 * 8);
    if (blocks > kStreamSinkWords) blocks = kStreamSinkWords;  // grid-stride beyond that
    if (blocks < 1) blocks = 1;
    stream_read_kernel<<<(int)blocks, 256, 0, s>>>(static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *h, int B, int d, float eps, float *n, hipStream_t s) {
    rmsnorm_kernel<<<B, 256, 0, s>>>(h, d, eps, n);
    return hipGetLastError();
}

// scale[b] = 1 / sqrt(mean(h_b^2) + eps), one workgroup per token, same
// summation order as the single-token predictor kernel's staging pass
__global__ __launch_bounds__(256) void rms_scale_kernel(const float *__restrict__ h, int d, float eps,
                                                        float *__restrict__ scale) {
    __shared__ float red[4];
    const float *hb = h + (size_t)blockIdx.x * d;
    constexpr int V = 8;
    const int nunits = d / 4;
    float ss = 0.0f;
    for (int base = threadIdx.x; base < nunits; base += blockDim.x * V) {
        float4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int m = base + u * (int)blockDim.x;
            if (m < nunits) v[u] = reinterpret_cast<const float4 *>(hb)[m];
        }
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int m = base + u * (int)blockDim.x;
            if (m < nunits) {
                ss = fmaf(v[u].x, v[u].x, ss);
                ss = fmaf(v[u].y, v[u].y, ss);
                ss = fmaf(v[u].z, v[u].z, ss);
                ss = fmaf(v[u].w, v[u].w, ss);
            }
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < 4; ++w) t += red[w];
        scale[blockIdx.x] = 1.0f / sqrtf(t / (float)d + eps);
    }
}

hipError_t launch_rms_scale(const float *h, int B, int d, float eps, float *scale, hipStream_t s) {
    rms_scale_kernel<<<B, 256, 0, s>>>(h, d, eps, scale);
    return hipGetLastError();
}

// y[e] = sum_{c < chunks} part[c * stride + e] (c ascending) (+ resid[e])
__global__ void reduce_kernel(const float *__restrict__ part, int chunks, int64_t stride,
                              const float *resid, float *y) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= stride) return;
    float s = 0.0f;
    for (int c = 0; c < chunks; ++c) s += part[c * stride + e];
    y[e] = resid ? resid[e] + s : s;
}

hipError_t launch_reduce(const float *part, int chunks, int B, int d, const float *resid,
                         float *y, hipStream_t s) {
    const int64_t n = (int64_t)B * d;
    reduce_kernel<<<(int)((n + 255) / 256), 256, 0, s>>>(part, chunks, n, resid, y);
    return hipGetLastError();
}

}  // namespace spffn
