// Single-token (batch 1) kernels, built for latency on gfx950: every wave
// issues its weight loads before anything that waits (LDS staging, the
// normalisation, barriers), so the 128-bit streaming loads overlap them.
//
// Decode step, per layer (four kernels):
//   w1_b1        hid = ReLU((W1 . h) * s + b1), s = 1/sqrt(mean(h^2) + eps)
//   pred2_up_b1  logit = W2 . hid + b2, mask = logit > t, and for the active
//                rows of each 8-row group act = max(z, 0) [* u] with
//                z = (W_act[i] . h) * s + b_i, listed per group
//   down_list_b1 part[c, slice] = sum over the lists of chunk c of
//                act * W_down_t[i, slice]
//   reduce_groups h = h + sum_c part[c]
// Single calls (spffn_predict / spffn_forward at one token): w1_b1, w2_b1
// (logits and mask), up_b1 (activations of an index list), down_b1 (partials
// over contiguous runs of the list), reduce_groups.
// (s is the RMS scale; multiplying the dot product by it equals normalising
// the vector first, up to rounding.)
#include <hip/hip_ext.h>

#include "device.h"

namespace spffn {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 128-bit streaming load: weights are read once per step, so they are marked
// non-temporal to leave the caches to activations, indices and partial sums.
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Stage one activation vector x[0..d) into the packet-transposed LDS layout
// (see device.h) with float4 loads, all of a thread's loads in flight at once;
// returns the thread's partial sum of squares (in a fixed order).
template <int E>
__device__ __forceinline__ float stage_vec(const float *__restrict__ x, int d, float *xl) {
    constexpr int V = 8;
    const int NP = d / E;
    const int nunits = d / 4;
    float ss = 0.0f;
    for (int base = threadIdx.x; base < nunits; base += blockDim.x * V) {
        float4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int m = base + u * (int)blockDim.x;
            if (m < nunits) v[u] = reinterpret_cast<const float4 *>(x)[m];
        }
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int m = base + u * (int)blockDim.x;
            if (m < nunits) {
                const int c = 4 * m, p = c / E, g = (c - p * E) >> 2;
                *reinterpret_cast<float4 *>(xl + (g * NP + p) * 4) = v[u];
                ss = fmaf(v[u].x, v[u].x, ss);
                ss = fmaf(v[u].y, v[u].y, ss);
                ss = fmaf(v[u].z, v[u].z, ss);
                ss = fmaf(v[u].w, v[u].w, ss);
            }
        }
    }
    return ss;
}

// Block-wide sum of one float per thread, same order in every block.
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += red[w];
    return t;
}

// ---------------------------------------------------------------------------
// predictor layer 1: one wave per row, 4 rows per block
// ---------------------------------------------------------------------------
template <int PF>
__global__ __launch_bounds__(256) void w1_b1_kernel(WMat w1, int r, int d,
                                                    const float *__restrict__ h, float eps,
                                                    int normalize, const float *__restrict__ b1,
                                                    float *__restrict__ hid,
                                                    float *__restrict__ scale_out) {
    constexpr int E = PacketElems<PF>::value;
    constexpr int U = 16;
    extern __shared__ float xl[];
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wv;
    const bool rv = row < r;
    const int NP = d / E;
    const uint4 *rp = row_ptr<PF>(w1, rv ? row : 0, d);

    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = u * 64 + lane;
        raw[u] = (rv && p < NP) ? ld_stream(rp + p) : make_uint4(0, 0, 0, 0);
    }
    const float ss = block_sum(stage_vec<E>(h, d, xl), red);  // contains the barrier
    const float s = normalize ? 1.0f / sqrtf(ss / (float)d + eps) : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out) *scale_out = s;

    float acc[1] = {0.0f};
    for (int pg = 0; pg < NP; pg += 64 * U) {
        if (pg > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = pg + u * 64 + lane;
                raw[u] = (rv && p < NP) ? ld_stream(rp + p) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = pg + u * 64 + lane;
            if (p < NP) packet_dot<PF, 1>(raw[u], 1.0f, xl, NP, p, nullptr, acc);
        }
    }
    const float v = wave_sum(acc[0]);
    if (rv && lane == 0) hid[row] = fmaxf(fmaf(v, s, b1 ? b1[row] : 0.0f), 0.0f);
}

// ---------------------------------------------------------------------------
// predictor layer 2 + threshold: R rows per wave, all their packets in flight
// ---------------------------------------------------------------------------
template <int PF, int R>
__global__ __launch_bounds__(256) void w2_b1_kernel(WMat w2, int rows, int r,
                                                    const float *__restrict__ hid,
                                                    const float *__restrict__ b2, float t,
                                                    float *__restrict__ logits,
                                                    uint8_t *__restrict__ mask) {
    constexpr int E = PacketElems<PF>::value;
    constexpr int PL = 2;  // packets per lane per row per pass
    extern __shared__ float xl[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wv) * R;
    const int NP = r / E;

    uint4 raw[R][PL];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int p = u * 64 + lane;
            raw[q][u] = (row0 + q < rows && p < NP)
                            ? ld_stream(row_ptr<PF>(w2, row0 + q, r) + p)
                            : make_uint4(0, 0, 0, 0);
        }
    stage_vec<E>(hid, r, xl);
    __syncthreads();

    float acc[R][1];
#pragma unroll
    for (int q = 0; q < R; ++q) acc[q][0] = 0.0f;
    for (int pg = 0; pg < NP; pg += 64 * PL) {
        if (pg > 0) {
#pragma unroll
            for (int q = 0; q < R; ++q)
#pragma unroll
                for (int u = 0; u < PL; ++u) {
                    const int p = pg + u * 64 + lane;
                    raw[q][u] = (row0 + q < rows && p < NP)
                                    ? ld_stream(row_ptr<PF>(w2, row0 + q, r) + p)
                                    : make_uint4(0, 0, 0, 0);
                }
        }
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int u = 0; u < PL; ++u) {
                const int p = pg + u * 64 + lane;
                if (p < NP) packet_dot<PF, 1>(raw[q][u], 1.0f, xl, NP, p, nullptr, acc[q]);
            }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float v = wave_sum(acc[q][0]);
        const int row = row0 + q;
        if (lane == 0 && row < rows) {
            const float l = v + b2[row];
            if (logits) logits[row] = l;
            mask[row] = (uint8_t)(l > t);
        }
    }
}

// ---------------------------------------------------------------------------
// row-gather gate/up GEMV + activation: one wave per listed neuron
// ---------------------------------------------------------------------------
struct UpB1Args {
    WMat wa, wu;
    const float *bias;
    int d, d_ffn;
    const int32_t *idx;    // nullptr: every neuron
    const int32_t *count;  // device count
    const float *h;        // [d]
    const float *scale;    // device RMS scale, or nullptr for 1
    float *act;            // [d_ffn], entry j of the list
};

template <int FMT, bool GATED, int U>
__global__ __launch_bounds__(256) void up_b1_kernel(UpB1Args a) {
    constexpr int E = PacketElems<FMT>::value;
    extern __shared__ float smem[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cnt = a.idx ? min(max(*a.count, 0), a.d_ffn) : a.d_ffn;
    if ((int)blockIdx.x * 4 >= cnt) return;  // block-uniform
    const int NP = a.d / E;
    float *xl = smem;
    float *xsum = smem + a.d;
    const int stride = gridDim.x * 4;

    int j = blockIdx.x * 4 + wv;
    int i = -1;
    if (j < cnt) i = a.idx ? a.idx[j] : j;
    bool valid = (i >= 0) && (i < a.d_ffn);

    uint4 ra[U], ru[U];
    float sa[U], su[U];
    auto load_group = [&](int pg) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = pg + u * 64 + lane;
            const bool ok = valid && p < NP;
            ra[u] = ok ? ld_stream(row_ptr<FMT>(a.wa, i, a.d) + p) : make_uint4(0, 0, 0, 0);
            sa[u] = ok ? packet_scale<FMT>(a.wa, i, a.d, p) : 0.0f;
            if constexpr (GATED) {
                ru[u] = ok ? ld_stream(row_ptr<FMT>(a.wu, i, a.d) + p) : make_uint4(0, 0, 0, 0);
                su[u] = ok ? packet_scale<FMT>(a.wu, i, a.d, p) : 0.0f;
            }
        }
    };
    load_group(0);
    stage_vec<E>(a.h, a.d, xl);
    if constexpr (FMT == kQ4) {
        __syncthreads();
        stage_xsum<E, 1>(xl, NP, xsum);
    }
    __syncthreads();
    const float s = a.scale ? *a.scale : 1.0f;

    for (;;) {
        float za[1] = {0.0f}, zu[1] = {0.0f};
        for (int pg = 0; pg < NP; pg += 64 * U) {
            if (pg > 0) load_group(pg);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = pg + u * 64 + lane;
                if (p < NP) {
                    packet_dot<FMT, 1>(ra[u], sa[u], xl, NP, p, xsum, za);
                    if constexpr (GATED) packet_dot<FMT, 1>(ru[u], su[u], xl, NP, p, xsum, zu);
                }
            }
        }
        if (j < cnt) {
            const float vz = wave_sum(za[0]);
            const float vu = GATED ? wave_sum(zu[0]) : 1.0f;
            if (lane == 0) {
                float v = 0.0f;
                if (valid) {
                    v = fmaxf(fmaf(vz, s, a.bias ? a.bias[i] : 0.0f), 0.0f);
                    if constexpr (GATED) v *= vu * s;
                }
                a.act[j] = v;
            }
        }
        j += stride;
        if (j >= cnt) break;
        i = a.idx ? a.idx[j] : j;
        valid = (i >= 0) && (i < a.d_ffn);
        load_group(0);
    }
}

// ---------------------------------------------------------------------------
// column-gather down projection: block (slice, chunk), one packet per lane
// ---------------------------------------------------------------------------
struct DownB1Args {
    WMat wd;
    int d, d_ffn;
    const int32_t *idx;
    const int32_t *count;
    const float *act;
    int chunks;
    float *part;  // [chunks, d]
};

template <int FMT, int UR>
__global__ __launch_bounds__(256) void down_b1_kernel(DownB1Args a) {
    constexpr int E = PacketElems<FMT>::value;
    __shared__ float red[64 * E];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, c = blockIdx.y;
    const int NP = a.d / E;
    const int p = slice * 64 + lane;
    const bool pv = p < NP;
    const int cnt = a.idx ? min(max(*a.count, 0), a.d_ffn) : a.d_ffn;
    const int per = (cnt + a.chunks - 1) / a.chunks;
    const int j0 = min(cnt, c * per), j1 = min(cnt, j0 + per);

    float acc[E], corr = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;

    // this wave's rows: j0 + wv + 4k; lanes prefetch up to 64 of them at once
    for (int kb = j0 + wv; kb < j1; kb += 4 * 64) {
        const int jl = kb + 4 * lane;
        int my_i = -1;
        float my_a = 0.0f;
        if (jl < j1) {
            const int ii = a.idx ? a.idx[jl] : jl;
            if (ii >= 0 && ii < a.d_ffn) {
                my_i = ii;
                my_a = a.act[jl];
            }
        }
        const int nk = min(64, (j1 - kb + 3) / 4);
        for (int k0 = 0; k0 < nk; k0 += UR) {
            uint4 raw[UR];
            float sc[UR], av[UR];
            int rowi[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                rowi[u] = __shfl(my_i, k0 + u, 64);
                av[u] = __shfl(my_a, k0 + u, 64);
                const bool ok = (k0 + u < nk) && rowi[u] >= 0 && pv;
                raw[u] = ok ? ld_stream(row_ptr<FMT>(a.wd, rowi[u], a.d) + p) : make_uint4(0, 0, 0, 0);
                sc[u] = ok ? packet_scale<FMT>(a.wd, rowi[u], a.d, p) : 0.0f;
                if (!ok) av[u] = 0.0f;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) packet_axpy<FMT>(raw[u], sc[u], av[u], acc, corr);
        }
    }

    packet_axpy_finish<FMT>(acc, corr);
    // fixed-order reduction of the four waves through LDS
    for (int w = 0; w < 4; ++w) {
        if (wv == w) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float &rr = red[lane * E + e];
                rr = (w == 0) ? acc[e] : rr + acc[e];
            }
        }
        __syncthreads();
    }
    const int col0 = slice * 64 * E;
    for (int t = threadIdx.x; t < 64 * E; t += blockDim.x)
        if (col0 + t < a.d) a.part[(size_t)c * a.d + col0 + t] = red[t];
}

// ---------------------------------------------------------------------------
// y[e] = sum_c part[c * n + e] (+ resid[e]): 32 columns x 8 chunk groups per
// block; each group sums its chunks in ascending order, then the groups are
// summed in a fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_groups_kernel(const float *__restrict__ part,
                                                            int chunks, int64_t n,
                                                            const float *resid, float *y,
                                                            const int32_t *__restrict__ ccnt,
                                                            int32_t *total_out) {
    __shared__ float red[8][33];
    const int col = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int64_t e = (int64_t)blockIdx.x * 32 + col;
    float s = 0.0f;
    if (e < n) {
        constexpr int V = 8;
        for (int c0 = g; c0 < chunks; c0 += 8 * V) {
            float v[V];
#pragma unroll
            for (int u = 0; u < V; ++u) {
                const int cc = c0 + 8 * u;
                v[u] = cc < chunks ? part[(int64_t)cc * n + e] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < V; ++u) s += v[u];
        }
    }
    red[g][col] = s;
    __syncthreads();
    if (g == 0 && e < n) {
        float tot = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) tot += red[k][col];
        y[e] = resid ? resid[e] + tot : tot;
    }
    // optional: total of the per-chunk row counts (first wave of block 0)
    if (total_out && blockIdx.x == 0 && threadIdx.x < 64) {
        int c = 0;
        for (int k = threadIdx.x; k < chunks; k += 64) c += ccnt[k];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
        if (threadIdx.x == 0) *total_out = c;
    }
}

// ---------------------------------------------------------------------------
// fused predictor layer 2 + threshold + gate/up gather (decode, one token)
//
// Workgroup g owns the interleaved W2 rows {g + G*k : k < RB} (G workgroups),
// so the hot-first rows spread one per workgroup.  It computes their logits,
// writes the mask, lists its active rows in LDS (ascending within the
// workgroup), and then computes the activation of each listed row with all
// four waves sharing the row's packets.  Output per workgroup g: all RB
// slots of its list in lst_i / lst_a (neuron, activation; its active rows
// first, the rest neuron -1).  The lists are stored
// chunk-major for the down projection: group g = c + C*j (C chunks) owns
// slots [(c*NG + j)*RB, +RB) with NG = ceil(G / C), so the lists of one chunk
// are contiguous and can be read without first reading the counts.
// ---------------------------------------------------------------------------
struct FusedArgs {
    WMat w2, wa, wu;
    int d, d_ffn, r;
    int groups;           // row groups of RB rows (rows interleaved with stride groups)
    const float *hid;     // [r]
    const float *b2;      // [d_ffn]
    float t;
    const float *bias;    // [d_ffn] or nullptr
    const float *h;       // [d] residual stream (un-normalised)
    const float *scale;   // device RMS scale
    float *logits;        // [d_ffn] or nullptr
    uint8_t *mask;        // [d_ffn]
    int32_t *lst_i;       // [C*NG*RB]
    float *lst_a;         // [C*NG*RB]
    int chunks;           // C: chunks of the down projection
    int per_chunk;        // NG = ceil(G / C): groups per chunk
};

template <int PF, int FMT, bool GATED, int RW, int UA>
__global__ __launch_bounds__(256) void pred2_up_b1_kernel(FusedArgs a) {
    constexpr int EP = PacketElems<PF>::value;
    constexpr int E = PacketElems<FMT>::value;
    constexpr int RB = 4 * RW;     // rows per row group (one group per workgroup)
    constexpr int PL = 2;          // W2 packets per lane per row (rows of <= 128 packets)
    __shared__ uint32_t s_bits[4];
    __shared__ int s_list[RB];     // listed rows, ascending
    __shared__ int s_loc[RB];      // their local index k in the group
    __shared__ float s_bias[RB];   // bias of every row of the group, by local index
    __shared__ float s_part[RB][4][2];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int G = a.groups, g = blockIdx.x;
    const int NPr = a.r / EP, NPd = a.d / E;

    // Everything the W2 phase needs is requested up front, straight into
    // registers: the wave's W2 rows g + G*(wv + 4q), the hid values of the
    // lane's two packets, the rows' b2 entries (lane q holds row q's) and the
    // bias of each of the group's rows (into LDS).  Addresses are clamped into
    // range and out-of-range values discarded, so the loads carry no branches.
    uint4 rc[RW][PL];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        const int row = g + G * (wv + 4 * q);
        const bool rv = row < a.d_ffn;
        const int rr = rv ? row : a.d_ffn - 1;
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int p = u * 64 + lane;
            const uint4 v = ld_stream(row_ptr<PF>(a.w2, rr, a.r) + (p < NPr ? p : NPr - 1));
            rc[q][u] = (rv && p < NPr) ? v : make_uint4(0, 0, 0, 0);
        }
    }
    float hv[PL][EP];
#pragma unroll
    for (int u = 0; u < PL; ++u) {
        const int p = u * 64 + lane;
        float unused;
        load_packet_x<PF>(a.hid, p < NPr ? p : NPr - 1, hv[u], unused);
    }
    float b2v;
    {
        const int row = g + G * (wv + 4 * (lane < RW ? lane : 0));
        b2v = a.b2[row < a.d_ffn ? row : a.d_ffn - 1];
    }
    if ((int)threadIdx.x < RB) {
        const int row = g + G * (int)threadIdx.x;
        s_bias[threadIdx.x] = (a.bias && row < a.d_ffn) ? a.bias[row] : 0.0f;
    }
    const float s = *a.scale;

    // logits, threshold, mask
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < PL; ++u)
            if (u * 64 + lane < NPr) acc = packet_dot_reg<PF>(rc[q][u], 1.0f, hv[u], 0.0f, acc);
        const float v = wave_sum(acc);
        const float bq = __shfl(b2v, q, 64);
        const int row = g + G * (wv + 4 * q);
        if (row < a.d_ffn) {
            const float l = v + bq;
            const bool m = l > a.t;
            bits |= (uint32_t)m << q;
            if (lane == 0) {
                if (a.logits) a.logits[row] = l;
                a.mask[row] = (uint8_t)m;
            }
        }
    }
    // list of the group's active rows, ordered by local index k = wv + 4q
    // (ascending row g + G*k)
    if (lane == 0) s_bits[wv] = bits;
    __syncthreads();
    int n_act = 0;
    for (int w = 0; w < 4; ++w) n_act += __popc(s_bits[w]);
    if (threadIdx.x < RB) {
        const int k = threadIdx.x, wk = k & 3, qk = k >> 2;
        if ((s_bits[wk] >> qk) & 1u) {
            int rank = 0;
            for (int k2 = 0; k2 < k; ++k2) rank += (s_bits[k2 & 3] >> (k2 >> 2)) & 1u;
            s_list[rank] = g + G * k;
            s_loc[rank] = k;
        }
    }
    __syncthreads();

    // activations of the listed rows: the four waves share each row, lane
    // (wv, lane) always takes packets wv*64 + lane + 256u, so its activation
    // values are loaded once, into registers, after the first row's weights
    // have been requested (a group without active rows never reads them)
    // Packets past the end of a row load a clamped (valid) packet and meet
    // zero activation values, so every load is unconditional.
    float xv[UA][E], xs[UA];
    for (int k = 0; k < n_act; ++k) {
        const int i = s_list[k];
        uint4 ra[UA], ru[UA];
        float sa[UA], su[UA];
#pragma unroll
        for (int u = 0; u < UA; ++u) {
            const int p = wv * 64 + lane + 256 * u;
            const int pc = p < NPd ? p : NPd - 1;
            ra[u] = ld_stream(row_ptr<FMT>(a.wa, i, a.d) + pc);
            sa[u] = packet_scale<FMT>(a.wa, i, a.d, pc);
            if constexpr (GATED) {
                ru[u] = ld_stream(row_ptr<FMT>(a.wu, i, a.d) + pc);
                su[u] = packet_scale<FMT>(a.wu, i, a.d, pc);
            }
        }
        if (k == 0) {
#pragma unroll
            for (int u = 0; u < UA; ++u) {
                const int p = wv * 64 + lane + 256 * u;
                load_packet_x<FMT>(a.h, p < NPd ? p : NPd - 1, xv[u], xs[u]);
            }
        }
        // keep every load of the row ahead of the first use (the scheduler
        // otherwise issues one load, waits for it, then issues the rest)
        __builtin_amdgcn_sched_barrier(0);
        if (k == 0) {
#pragma unroll
            for (int u = 0; u < UA; ++u)
                if (wv * 64 + lane + 256 * u >= NPd) {
#pragma unroll
                    for (int e = 0; e < E; ++e) xv[u][e] = 0.0f;
                    xs[u] = 0.0f;
                }
        }
        // no bounds branch here: out-of-range packets have zero activations,
        // and a branch lets the compiler sink their loads behind a full wait
        float za = 0.0f, zu = 0.0f;
#pragma unroll
        for (int u = 0; u < UA; ++u) {
            za = packet_dot_reg<FMT>(ra[u], sa[u], xv[u], xs[u], za);
            if constexpr (GATED) zu = packet_dot_reg<FMT>(ru[u], su[u], xv[u], xs[u], zu);
        }
        za = wave_sum(za);
        if constexpr (GATED) zu = wave_sum(zu);
        if (lane == 0) {
            s_part[k][wv][0] = za;
            s_part[k][wv][1] = zu;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < RB) {
        const int k = threadIdx.x;
        int row = -1;
        float v = 0.0f;
        if (k < n_act) {
            float vz = 0.0f, vu = 0.0f;
            for (int w = 0; w < 4; ++w) {
                vz += s_part[k][w][0];
                vu += s_part[k][w][1];
            }
            v = fmaxf(fmaf(vz, s, s_bias[s_loc[k]]), 0.0f);
            if constexpr (GATED) v *= vu * s;
            row = s_list[k];
        }
        const size_t slot = ((size_t)(g % a.chunks) * a.per_chunk + g / a.chunks) * RB + k;
        a.lst_i[slot] = row;
        a.lst_a[slot] = v;
    }
}

// ---------------------------------------------------------------------------
// down projection over the per-workgroup lists of the fused kernel: block
// (slice, chunk c) takes the lists of workgroups c, c + C, c + 2C, ... in that
// order.  Striding (rather than contiguous ranges) spreads the hot-first rows,
// which all sit in the first workgroups, evenly over the chunks.  The chunk's
// slots are contiguous, so every thread requests its share of them at once;
// the active ones (neuron >= 0) are compacted into LDS in slot order, and
// wave w then takes rows w, w + 4, w + 8, ... of that list.
// ---------------------------------------------------------------------------
struct DownListArgs {
    WMat wd;
    int d, d_ffn;
    const int32_t *lst_i;
    const float *lst_a;
    int G, RB;
    int chunks;
    int per_chunk;         // groups per chunk (slot stride of a chunk: per_chunk * RB)
    float *part;           // [chunks, d]
    int32_t *chunk_cnt;    // [chunks] rows listed per chunk, or nullptr
};

constexpr int kDownListMaxSlots = 64 * 20;  // groups per chunk <= 64, rows per group <= 20

template <int FMT, int UR>
__global__ __launch_bounds__(256) void down_list_b1_kernel(DownListArgs a) {
    constexpr int E = PacketElems<FMT>::value;
    constexpr int SPT = kDownListMaxSlots / 256;  // slots per thread
    __shared__ float red[64 * E];
    __shared__ int s_i[kDownListMaxSlots];
    __shared__ float s_a[kDownListMaxSlots];
    __shared__ int s_wc[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, c = blockIdx.y;
    const int NP = a.d / E;
    const int p = slice * 64 + lane;
    const bool pv = p < NP;
    const int C = a.chunks;
    const int ng = (a.G - c + C - 1) / C;  // groups c + C*j, j < ng; at most 64 (launcher)
    const int S = ng * a.RB;                // slots of this chunk
    const size_t base = (size_t)c * a.per_chunk * a.RB;

    int vi[SPT];
    float va[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int sl = (int)threadIdx.x + 256 * u;
        vi[u] = sl < S ? a.lst_i[base + sl] : -1;
        va[u] = sl < S ? a.lst_a[base + sl] : 0.0f;
    }
    // compaction of the active slots, in slot order
    int T = 0;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        if (256 * u >= S) break;  // block-uniform
        const bool act = vi[u] >= 0 && vi[u] < a.d_ffn;
        const unsigned long long bal = __ballot(act);
        if (lane == 0) s_wc[wv] = __popcll(bal);
        __syncthreads();
        int at = T;
        for (int w = 0; w < wv; ++w) at += s_wc[w];
        if (act) {
            const int q = at + __popcll(bal & below);
            s_i[q] = vi[u];
            s_a[q] = va[u];
        }
        T += s_wc[0] + s_wc[1] + s_wc[2] + s_wc[3];
        __syncthreads();
    }
    if (a.chunk_cnt && slice == 0 && threadIdx.x == 0) a.chunk_cnt[c] = T;

    float acc[E], corr = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;

    for (int fb = wv; fb < T; fb += 4 * UR) {
        // the batch's list entries first (clamped, so the LDS reads carry no
        // branches), then all of its row loads
        int ri[UR];
        float av[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int f = fb + 4 * u;
            const int fc = f < T ? f : T - 1;
            ri[u] = s_i[fc];
            av[u] = s_a[fc];
        }
        uint4 raw[UR];
        float sc[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const bool ok = fb + 4 * u < T && pv;
            raw[u] = make_uint4(0, 0, 0, 0);
            sc[u] = 0.0f;
            if (ok) {
                raw[u] = ld_stream(row_ptr<FMT>(a.wd, ri[u], a.d) + p);
                sc[u] = packet_scale<FMT>(a.wd, ri[u], a.d, p);
            } else {
                av[u] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) packet_axpy<FMT>(raw[u], sc[u], av[u], acc, corr);
    }

    packet_axpy_finish<FMT>(acc, corr);
    for (int w = 0; w < 4; ++w) {
        if (wv == w) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float &rr = red[lane * E + e];
                rr = (w == 0) ? acc[e] : rr + acc[e];
            }
        }
        __syncthreads();
    }
    const int col0 = slice * 64 * E;
    for (int t = threadIdx.x; t < 64 * E; t += blockDim.x)
        if (col0 + t < a.d) a.part[(size_t)c * a.d + col0 + t] = red[t];
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// The single-token kernels keep one activation vector in LDS.
bool b1_fits(const Layer &L) {
    const int d = L.desc.d;
    const int E = packet_elems(L.desc.w_dtype);
    const size_t lds = (size_t)d * 4 + (L.desc.w_dtype == SPFFN_Q4_0 ? (size_t)(d / E) * 4 : 0);
    return lds <= 56 * 1024 && (size_t)L.desc.r * 4 <= 56 * 1024;
}

hipError_t launch_w1_b1(const Layer &L, const float *h, float eps, bool normalize, float *hid,
                        float *scale_out, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    const int blocks = (D.r + 3) / 4;
    const size_t lds = (size_t)D.d * 4;
    if (D.p_dtype == SPFFN_F16)
        w1_b1_kernel<kF16><<<blocks, 256, lds, s>>>(L.w1, D.r, D.d, h, eps, normalize, D.p_b1, hid,
                                                    scale_out);
    else
        w1_b1_kernel<kF32><<<blocks, 256, lds, s>>>(L.w1, D.r, D.d, h, eps, normalize, D.p_b1, hid,
                                                    scale_out);
    return hipGetLastError();
}

hipError_t launch_w2_b1(const Layer &L, const float *hid, float *logits, uint8_t *mask,
                        hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    constexpr int R = 8;
    const int blocks = (D.d_ffn + 4 * R - 1) / (4 * R);
    const size_t lds = (size_t)D.r * 4;
    if (D.p_dtype == SPFFN_F16)
        w2_b1_kernel<kF16, R><<<blocks, 256, lds, s>>>(L.w2, D.d_ffn, D.r, hid, D.p_b2, L.t, logits,
                                                       mask);
    else
        w2_b1_kernel<kF32, R><<<blocks, 256, lds, s>>>(L.w2, D.d_ffn, D.r, hid, D.p_b2, L.t, logits,
                                                       mask);
    return hipGetLastError();
}

constexpr int kUpB1MaxBlocks = 1024;

hipError_t launch_up_b1(const Layer &L, const float *h, const float *scale, const int32_t *idx,
                        const int32_t *count, float *act, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    UpB1Args a{};
    const bool gated = D.kind == SPFFN_REGLU;
    a.wa = gated ? L.gate : L.up;
    a.wu = L.up;
    a.bias = D.b_act;
    a.d = D.d;
    a.d_ffn = D.d_ffn;
    a.idx = idx;
    a.count = count;
    a.h = h;
    a.scale = scale;
    a.act = act;
    int blocks = (D.d_ffn + 3) / 4;
    if (blocks > kUpB1MaxBlocks) blocks = kUpB1MaxBlocks;
    const int E = packet_elems(D.w_dtype);
    const size_t lds = (size_t)D.d * 4 + (D.w_dtype == SPFFN_Q4_0 ? (size_t)(D.d / E) * 4 : 0);
    switch (D.w_dtype) {
        case SPFFN_F32:
            if (gated) up_b1_kernel<kF32, true, 8><<<blocks, 256, lds, s>>>(a);
            else up_b1_kernel<kF32, false, 8><<<blocks, 256, lds, s>>>(a);
            break;
        case SPFFN_F16:
            if (gated) up_b1_kernel<kF16, true, 8><<<blocks, 256, lds, s>>>(a);
            else up_b1_kernel<kF16, false, 8><<<blocks, 256, lds, s>>>(a);
            break;
        default:
            if (gated) up_b1_kernel<kQ4, true, 4><<<blocks, 256, lds, s>>>(a);
            else up_b1_kernel<kQ4, false, 8><<<blocks, 256, lds, s>>>(a);
            break;
    }
    return hipGetLastError();
}

int down_b1_chunks(const Layer &L) {
    const int E = packet_elems(L.desc.w_dtype);
    const int slices = (L.desc.d / E + 63) / 64;
    int c = 2048 / slices;
    if (c > 64) c = 64;
    if (c < 16) c = 16;
    return c;
}

hipError_t launch_down_b1(const Layer &L, const int32_t *idx, const int32_t *count,
                          const float *act, float *part, int chunks, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    DownB1Args a{};
    a.wd = L.down;
    a.d = D.d;
    a.d_ffn = D.d_ffn;
    a.idx = idx;
    a.count = count;
    a.act = act;
    a.chunks = chunks;
    a.part = part;
    const int E = packet_elems(D.w_dtype);
    dim3 grid((D.d / E + 63) / 64, chunks);
    switch (D.w_dtype) {
        case SPFFN_F32: down_b1_kernel<kF32, 16><<<grid, 256, 0, s>>>(a); break;
        case SPFFN_F16: down_b1_kernel<kF16, 16><<<grid, 256, 0, s>>>(a); break;
        default: down_b1_kernel<kQ4, 8><<<grid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

// Row groups of the fused kernel: 8 rows per workgroup (two W2 rows per
// wave).  Small groups keep the kernel at 4-5 resident workgroups per CU and
// let the hardware hand new groups to CUs whose groups had few active rows,
// which balances the gather phase better than larger groups.
constexpr int kFusedRW = 2;
// 4-bit rows are 4.5x smaller than fp16 ones while every group with an active
// row still reads the whole fp32 activation vector (and its block sums), so
// their groups are larger (20 rows) to spread that read over more active rows
// (measured at the 175B-shaped layer: 8 rows 55.5 us, 12 rows 51.4, 16 rows
// 50.4-51.2, 20 rows 48.0-48.7, 24 rows 55.2, 28 rows 49.7, 32 rows 52.4).
constexpr int kFusedRWQ4 = 5;
static_assert(4 * kFusedRW * 64 <= kDownListMaxSlots && 4 * kFusedRWQ4 * 64 <= kDownListMaxSlots,
              "a down-projection chunk must hold its groups' list slots");

template <int FMT> constexpr int fused_rw() { return FMT == kQ4 ? kFusedRWQ4 : kFusedRW; }

int fused_rows_per_group(const Layer &L) {
    return 4 * (L.desc.w_dtype == SPFFN_Q4_0 ? kFusedRWQ4 : kFusedRW);
}
int fused_groups(const Layer &L) {
    const int RB = fused_rows_per_group(L);
    return (L.desc.d_ffn + RB - 1) / RB;
}

// Down-projection row chunks over the fused kernel's lists: at most 64 groups
// per chunk (one wave scans their counts), at least 64 chunks.
int fused_chunks(const Layer &L) {
    const int G = fused_groups(L);
    int c = (G + 63) / 64;
    if (c < 64) c = 64;
    return c < G ? c : G;
}

int fused_per_chunk(const Layer &L) {
    const int C = fused_chunks(L);
    return (fused_groups(L) + C - 1) / C;
}

size_t fused_list_slots(const Layer &L) {
    return (size_t)fused_chunks(L) * fused_per_chunk(L) * fused_rows_per_group(L);
}

// Activated-row packets per lane: one pass of 256*UA packets covers a row.
static int fused_ua(const Layer &L) {
    const int NPd = L.desc.d / packet_elems(L.desc.w_dtype);
    return NPd <= 512 ? 2 : NPd <= 1024 ? 4 : 8;
}

bool fused_fits(const Layer &L) {
    // a W2 row must fit one pass of 2 packets per lane, an activated row one
    // pass of 8 packets per lane
    return L.desc.r / packet_elems(L.desc.p_dtype) <= 128 &&
           L.desc.d / packet_elems(L.desc.w_dtype) <= 256 * 8;
}

template <int PF, int FMT, bool GATED, int RW, int UA>
static void launch_fused_t(const FusedArgs &a, int G, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    // with timing events the dispatch itself is timestamped (the events bracket
    // the kernel's execution, not its launch)
    if (e0 || e1)
        hipExtLaunchKernelGGL(pred2_up_b1_kernel<PF, FMT, GATED, RW, UA>, dim3(G), dim3(256), 0, s,
                              e0, e1, 0, a);
    else
        pred2_up_b1_kernel<PF, FMT, GATED, RW, UA><<<G, 256, 0, s>>>(a);
}

template <int PF, int FMT, bool GATED>
static void launch_fused_rw(const FusedArgs &a, int G, int UA, hipStream_t s, hipEvent_t e0,
                            hipEvent_t e1) {
    constexpr int RW = fused_rw<FMT>();
    if (UA == 2) launch_fused_t<PF, FMT, GATED, RW, 2>(a, G, s, e0, e1);
    else if (UA == 4) launch_fused_t<PF, FMT, GATED, RW, 4>(a, G, s, e0, e1);
    else launch_fused_t<PF, FMT, GATED, RW, 8>(a, G, s, e0, e1);
}

template <int PF, int FMT>
static void launch_fused_kind(const FusedArgs &a, bool gated, int G, int UA, hipStream_t s,
                              hipEvent_t e0, hipEvent_t e1) {
    if (gated) launch_fused_rw<PF, FMT, true>(a, G, UA, s, e0, e1);
    else launch_fused_rw<PF, FMT, false>(a, G, UA, s, e0, e1);
}

hipError_t launch_pred2_up_b1(const Layer &L, const float *hid, const float *h, const float *scale,
                              float *logits, uint8_t *mask, int32_t *lst_i, float *lst_a,
                              hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    const spffn_layer_desc &D = L.desc;
    FusedArgs a{};
    const bool gated = D.kind == SPFFN_REGLU;
    a.w2 = L.w2;
    a.wa = gated ? L.gate : L.up;
    a.wu = L.up;
    a.d = D.d;
    a.d_ffn = D.d_ffn;
    a.r = D.r;
    a.hid = hid;
    a.b2 = D.p_b2;
    a.t = L.t;
    a.bias = D.b_act;
    a.h = h;
    a.scale = scale;
    a.logits = logits;
    a.mask = mask;
    a.lst_i = lst_i;
    a.lst_a = lst_a;
    const int G = fused_groups(L), UA = fused_ua(L);
    a.groups = G;
    a.chunks = fused_chunks(L);
    a.per_chunk = fused_per_chunk(L);
    if (D.p_dtype == SPFFN_F16) {
        if (D.w_dtype == SPFFN_F16) launch_fused_kind<kF16, kF16>(a, gated, G, UA, s, ev_start, ev_stop);
        else if (D.w_dtype == SPFFN_F32) launch_fused_kind<kF16, kF32>(a, gated, G, UA, s, ev_start, ev_stop);
        else launch_fused_kind<kF16, kQ4>(a, gated, G, UA, s, ev_start, ev_stop);
    } else {
        if (D.w_dtype == SPFFN_F16) launch_fused_kind<kF32, kF16>(a, gated, G, UA, s, ev_start, ev_stop);
        else if (D.w_dtype == SPFFN_F32) launch_fused_kind<kF32, kF32>(a, gated, G, UA, s, ev_start, ev_stop);
        else launch_fused_kind<kF32, kQ4>(a, gated, G, UA, s, ev_start, ev_stop);
    }
    return hipGetLastError();
}

hipError_t launch_down_list_b1(const Layer &L, const int32_t *lst_i, const float *lst_a,
                               float *part, int chunks, int32_t *chunk_cnt, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    // the fused kernel laid its lists out for exactly fused_chunks(L) chunks
    if (chunks != fused_chunks(L)) return hipErrorInvalidValue;
    DownListArgs a{};
    a.wd = L.down;
    a.d = D.d;
    a.d_ffn = D.d_ffn;
    a.lst_i = lst_i;
    a.lst_a = lst_a;
    a.G = fused_groups(L);
    a.RB = fused_rows_per_group(L);
    a.chunks = chunks;
    a.per_chunk = fused_per_chunk(L);
    a.part = part;
    a.chunk_cnt = chunk_cnt;
    const int E = packet_elems(D.w_dtype);
    dim3 grid((D.d / E + 63) / 64, chunks);
    switch (D.w_dtype) {
        case SPFFN_F32: down_list_b1_kernel<kF32, 16><<<grid, 256, 0, s>>>(a); break;
        case SPFFN_F16: down_list_b1_kernel<kF16, 16><<<grid, 256, 0, s>>>(a); break;
        default: down_list_b1_kernel<kQ4, 8><<<grid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t launch_reduce_groups(const float *part, int chunks, int64_t n, const float *resid,
                                float *y, hipStream_t s, const int32_t *chunk_cnt,
                                int32_t *total_out) {
    reduce_groups_kernel<<<(int)((n + 31) / 32), 256, 0, s>>>(part, chunks, n, resid, y, chunk_cnt,
                                                              total_out);
    return hipGetLastError();
}

}  // namespace spffn
