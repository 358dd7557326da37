// Neuron-sparse FFN kernels: row-gather gate/up GEMV with the activation, and
// the column-gather down projection into per-chunk partial sums.
//
// Up:   for every listed neuron j (i = idx[j], or i = j when dense) one wave
//       streams row i of the activated matrix (and of W_up when gated) as
//       16-byte packets against x staged in LDS, then writes
//       act[b, j] = max(z, 0) (ReLU) or max(z, 0) * u (ReGLU).
// Down: the listed rows of W_down_t are split into `chunks` contiguous runs of
//       the index list; block (s, c) owns packet column s (64 packets per
//       slice) and run c, accumulates act[b, j] * W_down_t[i, slice] over its
//       run, reduces its waves in a fixed order through LDS and writes
//       part[c, b, slice].  A separate pass sums the chunks in ascending order,
//       so results do not depend on scheduling (no atomics carry data).
#include "device.h"

namespace spffn {

constexpr int kUpWaves = 4;
constexpr int kDownWaves = 4;

struct UpArgs {
    WMat wa;            // activated projection (gate for ReGLU, up for ReLU)
    WMat wu;            // W_up for ReGLU
    const float *bias;  // [d_ffn] or nullptr
    int d, d_ffn;
    const int32_t *idx;    // [count] or nullptr (dense)
    const int32_t *count;  // device count (ignored when dense)
    const float *x;        // [B, d]
    int B;
    float *act;  // [B, d_ffn] (row stride d_ffn), entry j of the list
    int chunk_packets;
    bool silu;   // SwiGLU: SiLU instead of ReLU on the gate
};

template <int FMT, int NB, bool GATED, int U>
__global__ __launch_bounds__(kUpWaves * kWave) void ffn_up_kernel(UpArgs a) {
    constexpr int E = PacketElems<FMT>::value;
    extern __shared__ float smem[];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int cnt = a.idx ? min(max(*a.count, 0), a.d_ffn) : a.d_ffn;
    if ((int)(blockIdx.x * kUpWaves) >= cnt) return;  // block-uniform

    const int NPtot = a.d / E;
    const int NPc = a.chunk_packets;
    const int nchunks = (NPtot + NPc - 1) / NPc;
    float *xl = smem;
    float *xsum = smem + NB * NPc * E;

    if (nchunks == 1) {
        stage_x<E, NB>(a.x, a.B, a.d, 0, NPtot, xl);
        if constexpr (FMT == kQ4) {
            __syncthreads();
            stage_xsum<E, NB>(xl, NPtot, xsum);
        }
        __syncthreads();
    }

    for (int jb = blockIdx.x * kUpWaves; jb < cnt; jb += gridDim.x * kUpWaves) {
        const int j = jb + wv;
        int i = -1;
        if (j < cnt) i = a.idx ? a.idx[j] : j;
        const bool valid = (i >= 0) && (i < a.d_ffn);
        float za[NB], zu[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) za[b] = zu[b] = 0.0f;

        for (int ch = 0; ch < nchunks; ++ch) {
            const int p0 = ch * NPc;
            const int np = min(NPc, NPtot - p0);
            if (nchunks > 1) {
                __syncthreads();
                stage_x<E, NB>(a.x, a.B, a.d, p0 * E, np, xl);
                if constexpr (FMT == kQ4) {
                    __syncthreads();
                    stage_xsum<E, NB>(xl, np, xsum);
                }
                __syncthreads();
            }
            if (!valid) continue;
            const uint4 *ra = row_ptr<FMT>(a.wa, i, a.d) + p0;
            const uint4 *ru = GATED ? row_ptr<FMT>(a.wu, i, a.d) + p0 : nullptr;
            for (int pb = 0; pb < np; pb += kWave * U) {
                uint4 rawa[U], rawu[U];
                float sa[U], su[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int p = pb + u * kWave + lane;
                    if (p < np) {
                        rawa[u] = ra[p];
                        sa[u] = packet_scale<FMT>(a.wa, i, a.d, p0 + p);
                        if constexpr (GATED) {
                            rawu[u] = ru[p];
                            su[u] = packet_scale<FMT>(a.wu, i, a.d, p0 + p);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int p = pb + u * kWave + lane;
                    if (p < np) {
                        packet_dot<FMT, NB>(rawa[u], sa[u], xl, np, p, xsum, za);
                        if constexpr (GATED) packet_dot<FMT, NB>(rawu[u], su[u], xl, np, p, xsum, zu);
                    }
                }
            }
        }
        if (j < cnt) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                za[b] = wave_sum(za[b]);
                if constexpr (GATED) zu[b] = wave_sum(zu[b]);
            }
            if (lane == 0) {
                const float bias = (valid && a.bias) ? a.bias[i] : 0.0f;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < a.B) {
                        float v = gate_act(za[b] + bias, a.silu);
                        if constexpr (GATED) v *= zu[b];
                        a.act[(size_t)b * a.d_ffn + j] = valid ? v : 0.0f;
                    }
                }
            }
        }
    }
}

struct DownArgs {
    WMat wd;  // W_down_t [d_ffn, d]
    int d, d_ffn;
    const int32_t *idx;
    const int32_t *count;
    const float *act;  // [B, d_ffn]
    int B;             // tokens in the whole batch (act / part row count)
    int b0, nb;        // token range of this launch
    int chunks;
    float *part;  // [chunks, B, d]
};

template <int FMT, int NB, int U>
__global__ __launch_bounds__(kDownWaves * kWave) void ffn_down_kernel(DownArgs a) {
    constexpr int E = PacketElems<FMT>::value;
    __shared__ float red[NB * kWave * E];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int slice = blockIdx.x, c = blockIdx.y;
    const int NPtot = a.d / E;
    const int p = slice * kWave + lane;
    const bool pvalid = p < NPtot;
    const int cnt = a.idx ? min(max(*a.count, 0), a.d_ffn) : a.d_ffn;
    const int per = (cnt + a.chunks - 1) / a.chunks;
    const int j0 = min(cnt, c * per), j1 = min(cnt, j0 + per);

    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.0f;

    for (int jb = j0 + wv; jb < j1; jb += kDownWaves * U) {
        uint4 raw[U];
        float sc[U];
        int ii[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jb + u * kDownWaves;
            int i = -1;
            if (j < j1) i = a.idx ? a.idx[j] : j;
            ii[u] = (i >= 0 && i < a.d_ffn) ? i : -1;
            if (ii[u] >= 0 && pvalid) {
                raw[u] = row_ptr<FMT>(a.wd, ii[u], a.d)[p];
                sc[u] = packet_scale<FMT>(a.wd, ii[u], a.d, p);
            } else {
                raw[u] = make_uint4(0, 0, 0, 0);
                sc[u] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jb + u * kDownWaves;
            if (ii[u] < 0) continue;
            float w[E];
            packet_values<FMT>(raw[u], sc[u], w);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b < a.nb) {
                    const float av = a.act[(size_t)(a.b0 + b) * a.d_ffn + j];
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[b][e] = fmaf(av, w[e], acc[b][e]);
                }
            }
        }
    }

    // fixed-order reduction of the block's waves: wave 0, then 1, 2, 3
    for (int w = 0; w < kDownWaves; ++w) {
        if (wv == w) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float &r = red[(b * kWave + lane) * E + e];
                    r = (w == 0) ? acc[b][e] : r + acc[b][e];
                }
        }
        __syncthreads();
    }
    const int slice_cols = kWave * E;
    const int col0 = slice * slice_cols;
    for (int t = threadIdx.x; t < NB * slice_cols; t += blockDim.x) {
        const int b = t / slice_cols, k = t - b * slice_cols;
        const int col = col0 + k;
        if (b < a.nb && col < a.d)
            a.part[((size_t)c * a.B + a.b0 + b) * a.d + col] = red[t];
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
constexpr int kLdsBudgetUp = 56 * 1024;

int down_chunks(const Layer &L) {
    const int E = packet_elems(L.desc.w_dtype);
    const int slices = (L.desc.d / E + kWave - 1) / kWave;
    int c = 1024 / slices;
    if (c > 64) c = 64;
    if (c < 1) c = 1;
    return c;
}

template <int FMT, int NB>
static hipError_t up_dispatch(const Layer &L, UpArgs &a, hipStream_t s) {
    constexpr int E = PacketElems<FMT>::value;
    const int per_packet = NB * E * 4 + (FMT == kQ4 ? NB * 4 : 0);
    const int tot = a.d / E;
    a.chunk_packets = kLdsBudgetUp / per_packet < tot ? kLdsBudgetUp / per_packet : tot;
    const size_t lds = (size_t)a.chunk_packets * per_packet;
    int blocks = (a.d_ffn + kUpWaves - 1) / kUpWaves;
    if (blocks > 2048) blocks = 2048;
    if (L.desc.kind != SPFFN_RELU)
        ffn_up_kernel<FMT, NB, true, 4><<<blocks, kUpWaves * kWave, lds, s>>>(a);
    else
        ffn_up_kernel<FMT, NB, false, 8><<<blocks, kUpWaves * kWave, lds, s>>>(a);
    return hipGetLastError();
}

template <int FMT>
static hipError_t up_dispatch_nb(const Layer &L, UpArgs &a, hipStream_t s) {
    if (a.B <= 1) return up_dispatch<FMT, 1>(L, a, s);
    if (a.B <= 2) return up_dispatch<FMT, 2>(L, a, s);
    if (a.B <= 4) return up_dispatch<FMT, 4>(L, a, s);
    if (a.B <= 8) return up_dispatch<FMT, 8>(L, a, s);
    return up_dispatch<FMT, 16>(L, a, s);
}

hipError_t launch_ffn_up(const Layer &L, const float *x, int B, const int32_t *idx,
                         const int32_t *count, float *act, hipStream_t s) {
    UpArgs a{};
    const bool gated = L.desc.kind != SPFFN_RELU;
    a.wa = gated ? L.gate : L.up;
    a.wu = L.up;
    a.bias = L.desc.b_act;
    a.silu = L.desc.kind == SPFFN_SWIGLU;
    a.d = L.desc.d;
    a.d_ffn = L.desc.d_ffn;
    a.idx = idx;
    a.count = count;
    a.x = x;
    a.B = B;
    a.act = act;
    switch (L.desc.w_dtype) {
        case SPFFN_F32: return up_dispatch_nb<kF32>(L, a, s);
        case SPFFN_F16: return up_dispatch_nb<kF16>(L, a, s);
        default: return up_dispatch_nb<kQ4>(L, a, s);
    }
}

template <int FMT, int NB>
static hipError_t down_launch(DownArgs &a, hipStream_t s) {
    constexpr int E = PacketElems<FMT>::value;
    const int slices = (a.d / E + kWave - 1) / kWave;
    dim3 grid(slices, a.chunks);
    ffn_down_kernel<FMT, NB, 4><<<grid, kDownWaves * kWave, 0, s>>>(a);
    return hipGetLastError();
}

template <int FMT>
static hipError_t down_dispatch_nb(DownArgs &a, hipStream_t s) {
    if (a.nb <= 1) return down_launch<FMT, 1>(a, s);
    if (a.nb <= 2) return down_launch<FMT, 2>(a, s);
    if (a.nb <= 4) return down_launch<FMT, 4>(a, s);
    if (a.nb <= 8) return down_launch<FMT, 8>(a, s);
    return down_launch<FMT, 16>(a, s);
}

hipError_t launch_ffn_down(const Layer &L, int B, const int32_t *idx, const int32_t *count,
                           const float *act, float *part, int chunks, hipStream_t s) {
    DownArgs a{};
    a.wd = L.down;
    a.d = L.desc.d;
    a.d_ffn = L.desc.d_ffn;
    a.idx = idx;
    a.count = count;
    a.act = act;
    a.B = B;
    a.chunks = chunks;
    a.part = part;
    if (L.desc.w_dtype == SPFFN_Q4_0) {
        // 32 accumulators per token and lane: two tokens per launch
        for (int b0 = 0; b0 < B; b0 += 2) {
            a.b0 = b0;
            a.nb = B - b0 < 2 ? B - b0 : 2;
            hipError_t e = a.nb == 1 ? down_launch<kQ4, 1>(a, s) : down_launch<kQ4, 2>(a, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    a.b0 = 0;
    a.nb = B;
    return L.desc.w_dtype == SPFFN_F32 ? down_dispatch_nb<kF32>(a, s)
                                       : down_dispatch_nb<kF16>(a, s);
}

}  // namespace spffn
