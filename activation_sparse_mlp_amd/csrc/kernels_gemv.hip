// Dense row GEMVs: the two predictor layers and the activation profile.
//
// One launch computes W[row] . x_b for every row and for a batch of NB tokens
// (B <= NB real ones).  Rows are streamed once as 16-byte packets; x is staged
// in LDS (packet-transposed, see device.h), in column chunks when the batch
// does not fit.  KS waves share a row when rows are long (each takes every
// KS-th run of 64 packets) and one wave takes R rows when rows are short, so
// every lane keeps several 128-bit loads in flight.
#include "device.h"

namespace spffn {

enum Epi : int { kEpiHid = 0, kEpiMask = 1, kEpiCount = 2 };

struct GemvArgs {
    WMat w;
    int rows, cols;
    const float *x;   // [B, cols]
    int B;
    const float *bias;  // [rows] or nullptr
    float t;
    const float *tvec;  // kEpiMask: per-token thresholds [B] replacing t, or nullptr
    int kd;             // kEpiMask: rows [0, kd) always active (logit reported +inf)
    float *out;         // kEpiHid: [B, rows]
    float *logits;      // kEpiMask: [B, rows] or nullptr
    uint8_t *mask;      // kEpiMask: [B, rows] or nullptr
    uint8_t *uni;       // kEpiMask: [rows] or nullptr
    int32_t *counts;    // kEpiCount: [rows]
    int chunk_packets;  // packets per LDS chunk
};

constexpr int kGemvWaves = 4;

template <int EPI, int NB>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs &a, int row, const float (&v)[NB]) {
    const float bias = a.bias ? a.bias[row] : 0.0f;
    if constexpr (EPI == kEpiHid) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < a.B) a.out[(size_t)b * a.rows + row] = fmaxf(v[b] + bias, 0.0f);
    } else if constexpr (EPI == kEpiMask) {
        uint8_t u = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < a.B) {
                const bool pre = row < a.kd;
                const float l = pre ? __builtin_inff() : v[b] + bias;
                const uint8_t m = (uint8_t)(pre || l > (a.tvec ? a.tvec[b] : a.t));
                if (a.logits) a.logits[(size_t)b * a.rows + row] = l;
                if (a.mask) a.mask[(size_t)b * a.rows + row] = m;
                u |= m;
            }
        }
        if (a.uni) a.uni[row] = u;
    } else {
        int c = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < a.B) c += (v[b] + bias > 0.0f);
        a.counts[row] += c;
    }
}

template <int FMT, int NB, int R, int KS, int U, int EPI>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_kernel(GemvArgs a) {
    constexpr int E = PacketElems<FMT>::value;
    constexpr int G = kGemvWaves / KS;  // row groups per block
    extern __shared__ float smem[];
    __shared__ float red[kGemvWaves][R][NB];

    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int grp = wv / KS, q = wv % KS;
    const int NPtot = a.cols / E;
    const int NPc = a.chunk_packets;
    const int nchunks = (NPtot + NPc - 1) / NPc;
    float *xl = smem;
    float *xsum = smem + NB * NPc * E;
    const int rows_per_block = G * R;

    if (nchunks == 1) {
        stage_x<E, NB>(a.x, a.B, a.cols, 0, NPtot, xl);
        if constexpr (FMT == kQ4) {
            __syncthreads();
            stage_xsum<E, NB>(xl, NPtot, xsum);
        }
        __syncthreads();
    }

    for (int row0 = blockIdx.x * rows_per_block; row0 < a.rows;
         row0 += gridDim.x * rows_per_block) {
        const int myrow0 = row0 + grp * R;
        float acc[R][NB];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;

        for (int ch = 0; ch < nchunks; ++ch) {
            const int p0 = ch * NPc;
            const int np = min(NPc, NPtot - p0);
            if (nchunks > 1) {
                __syncthreads();
                stage_x<E, NB>(a.x, a.B, a.cols, p0 * E, np, xl);
                if constexpr (FMT == kQ4) {
                    __syncthreads();
                    stage_xsum<E, NB>(xl, np, xsum);
                }
                __syncthreads();
            }
            for (int pb = q * kWave; pb < np; pb += KS * kWave * U) {
                uint4 raw[R][U];
                float sc[R][U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int p = pb + u * KS * kWave + lane;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int row = myrow0 + r;
                        if (p < np && row < a.rows) {
                            raw[r][u] = row_ptr<FMT>(a.w, row, a.cols)[p0 + p];
                            sc[r][u] = packet_scale<FMT>(a.w, row, a.cols, p0 + p);
                        } else {
                            raw[r][u] = make_uint4(0, 0, 0, 0);
                            sc[r][u] = 0.0f;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int p = pb + u * KS * kWave + lane;
                    if (p < np) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            packet_dot<FMT, NB>(raw[r][u], sc[r][u], xl, np, p, xsum, acc[r]);
                    }
                }
            }
        }

#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);

        if constexpr (KS == 1) {
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (myrow0 + r < a.rows) gemv_epilogue<EPI, NB>(a, myrow0 + r, acc[r]);
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < NB; ++b) red[wv][r][b] = acc[r][b];
            }
            __syncthreads();
            if ((int)threadIdx.x < G * R) {
                const int g = threadIdx.x / R, r = threadIdx.x % R;
                const int row = row0 + g * R + r;
                float v[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float s = 0.0f;
#pragma unroll
                    for (int k = 0; k < KS; ++k) s += red[g * KS + k][r][b];
                    v[b] = s;
                }
                if (row < a.rows) gemv_epilogue<EPI, NB>(a, row, v);
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
constexpr int kLdsBudget = 56 * 1024;  // dynamic LDS; static arrays fit beside it

static int gemv_chunk_packets(int fmt, int NB, int cols) {
    const int E = packet_elems(fmt);
    const int per_packet = NB * E * 4 + (fmt == kQ4 ? NB * 4 : 0);
    int np = kLdsBudget / per_packet;
    const int tot = cols / E;
    return np < tot ? np : tot;
}

template <int FMT, int NB, int EPI>
static hipError_t gemv_dispatch_shape(GemvArgs &a, hipStream_t s) {
    a.chunk_packets = gemv_chunk_packets(FMT, NB, a.cols);
    const size_t lds = (size_t)a.chunk_packets * (NB * PacketElems<FMT>::value * 4 +
                                                  (FMT == kQ4 ? NB * 4 : 0));
    const bool long_rows = row_bytes<FMT>(a.cols) >= 4096;
    if (long_rows) {
        constexpr int R = 1, KS = 4, U = 4;
        const int rpb = (kGemvWaves / KS) * R;
        const int blocks = (a.rows + rpb - 1) / rpb;
        gemv_kernel<FMT, NB, R, KS, U, EPI><<<blocks, kGemvWaves * kWave, lds, s>>>(a);
    } else {
        constexpr int R = 4, KS = 1, U = 2;
        const int rpb = (kGemvWaves / KS) * R;
        const int blocks = (a.rows + rpb - 1) / rpb;
        gemv_kernel<FMT, NB, R, KS, U, EPI><<<blocks, kGemvWaves * kWave, lds, s>>>(a);
    }
    return hipGetLastError();
}

template <int FMT, int EPI>
static hipError_t gemv_dispatch_nb(GemvArgs &a, hipStream_t s) {
    if (a.B <= 1) return gemv_dispatch_shape<FMT, 1, EPI>(a, s);
    if (a.B <= 2) return gemv_dispatch_shape<FMT, 2, EPI>(a, s);
    if (a.B <= 4) return gemv_dispatch_shape<FMT, 4, EPI>(a, s);
    if (a.B <= 8) return gemv_dispatch_shape<FMT, 8, EPI>(a, s);
    return gemv_dispatch_shape<FMT, 16, EPI>(a, s);
}

template <int EPI>
static hipError_t gemv_dispatch_fp(int fmt, GemvArgs &a, hipStream_t s) {
    if (fmt == kF32) return gemv_dispatch_nb<kF32, EPI>(a, s);
    if (fmt == kF16) return gemv_dispatch_nb<kF16, EPI>(a, s);
    if (fmt == kFP8) return gemv_dispatch_nb<kFP8, EPI>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_hid(int fmt, WMat w, int rows, int cols, const float *x, int B,
                           const float *bias, float *out, hipStream_t s) {
    GemvArgs a{};
    a.w = w;
    a.rows = rows;
    a.cols = cols;
    a.x = x;
    a.B = B;
    a.bias = bias;
    a.out = out;
    return gemv_dispatch_fp<kEpiHid>(fmt, a, s);
}

hipError_t launch_gemv_mask(int fmt, WMat w, int rows, int cols, const float *x, int B,
                            const float *bias, float t, const float *tvec, int kd,
                            float *logits, uint8_t *mask, uint8_t *uni, hipStream_t s) {
    GemvArgs a{};
    a.w = w;
    a.rows = rows;
    a.cols = cols;
    a.x = x;
    a.B = B;
    a.bias = bias;
    a.t = t;
    a.tvec = tvec;
    a.kd = kd;
    a.logits = logits;
    a.mask = mask;
    a.uni = uni;
    return gemv_dispatch_fp<kEpiMask>(fmt, a, s);
}

hipError_t launch_gemv_count(int fmt, WMat w, int rows, int cols, const float *x, int B,
                             const float *bias, int32_t *counts, hipStream_t s) {
    // tokens go in groups of 16 (one launch each); counts accumulate in order
    for (int b0 = 0; b0 < B; b0 += 16) {
        GemvArgs a{};
        a.w = w;
        a.rows = rows;
        a.cols = cols;
        a.x = x + (size_t)b0 * cols;
        a.B = B - b0 < 16 ? B - b0 : 16;
        a.bias = bias;
        a.counts = counts;
        hipError_t e;
        if (fmt == kF32)
            e = gemv_dispatch_shape<kF32, 16, kEpiCount>(a, s);
        else if (fmt == kF16)
            e = gemv_dispatch_shape<kF16, 16, kEpiCount>(a, s);
        else
            e = gemv_dispatch_shape<kQ4, 16, kEpiCount>(a, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace spffn
