// Single-token (batch 1) kernels, built for latency on gfx950: every wave
// issues its weight loads before anything that waits (LDS staging, the
// normalisation, barriers), so the 128-bit streaming loads overlap them.
//
// Decode step, per layer (three kernels):
//   w1x_b1       hid = ReLU((W1 . h) * s + b1), s = 1/sqrt(mean(h^2) + eps)
//   layer_b1     row groups: logit = W2 . hid + b2, mask = logit > t, and for
//                the active rows of each row group act = max(z, 0) [* u]
//                with z = (W_act[i] . h) * s + b_i, listed per group;
//                down workgroups (same launch, once a chunk's groups are
//                done): part[c, slice] = sum over the lists of chunk c of
//                act * W_down_t[i, slice]
//   reduce_groups h = h + sum_c part[c]
// Single calls (spffn_predict / spffn_forward at one token): w1x_b1, w2_b1
// (logits and mask), up_b1 (activations of an index list), down_b1 (partials
// over contiguous runs of the list), reduce_groups.
// (s is the RMS scale; multiplying the dot product by it equals normalising
// the vector first, up to rounding.)
#include <hip/hip_ext.h>

#include <atomic>

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

// ---------------------------------------------------------------------------
// predictor layer 1, activations in registers: RB rows per block, thread t
// takes packets t + 256u of every row (coalesced), with the activation values
// of those packets loaded once into registers; block-wide sums in a fixed
// order.  Every block also sums h^2 over the whole vector in the same order,
// so all of them use the same RMS scale.
// ---------------------------------------------------------------------------
template <int PF, int RB, int UB>
__global__ __launch_bounds__(256) void w1x_b1_kernel(WMat w1, int r, int d,
                                                     const float *__restrict__ h, float eps,
                                                     int normalize, const float *__restrict__ b1,
                                                     float *__restrict__ hid,
                                                     float *__restrict__ scale_out,
                                                     const float *__restrict__ tvec, float t) {
    constexpr int E = PacketElems<PF>::value;  // UB: packets per thread per pass
    __shared__ float s_red[4][RB + 1];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int NP = d / E;
    const int r0 = blockIdx.x * RB;
    const uint4 *q[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) q[k] = row_ptr<PF>(w1, min(r0 + k, r - 1), d);
    float acc[RB], ss = 0.0f;
#pragma unroll
    for (int k = 0; k < RB; ++k) acc[k] = 0.0f;
    for (int pb = 0; pb < NP; pb += 256 * UB) {
        uint4 w[RB][UB];
        float xv[UB][E];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int p = pb + (int)threadIdx.x + 256 * u;
            const int pc = p < NP ? p : NP - 1;
#pragma unroll
            for (int k = 0; k < RB; ++k) w[k][u] = ld_stream(q[k] + pc);
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int p = pb + (int)threadIdx.x + 256 * u;
            float unused;
            load_packet_x<PF>(h, p < NP ? p : NP - 1, xv[u], unused);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            // packets past the end of the rows meet zero activations
            if (pb + (int)threadIdx.x + 256 * u >= NP) {
#pragma unroll
                for (int e = 0; e < E; ++e) xv[u][e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) ss = fmaf(xv[u][e], xv[u][e], ss);
#pragma unroll
            for (int k = 0; k < RB; ++k) acc[k] = packet_dot_reg<PF>(w[k][u], 1.0f, xv[u], 0.0f, acc[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) acc[k] = wave_sum(acc[k]);
    ss = wave_sum(ss);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < RB; ++k) s_red[wv][k] = acc[k];
        s_red[wv][RB] = ss;
    }
    __syncthreads();
    if ((int)threadIdx.x <= RB) {
        const int k = threadIdx.x;
        const float sst = ((s_red[0][RB] + s_red[1][RB]) + s_red[2][RB]) + s_red[3][RB];
        const float s = normalize ? 1.0f / sqrtf(sst / (float)d + eps) : 1.0f;
        if (k < RB) {
            const int row = r0 + k;
            if (row < r) {
                const float tot = ((s_red[0][k] + s_red[1][k]) + s_red[2][k]) + s_red[3][k];
                hid[row] = fmaxf(fmaf(tot * row_scale<PF>(w1, row), s, b1 ? b1[row] : 0.0f), 0.0f);
            }
        } else if (blockIdx.x == 0 && scale_out) {
            // scale_out[0] = the RMS scale, scale_out[1] = the token's logit
            // threshold (its own, or the layer's): the layer kernel reads both
            scale_out[0] = s;
            scale_out[1] = tvec ? *tvec : t;
        }
    }
}

// ---------------------------------------------------------------------------
// predictor layer 2 + threshold: R rows per wave, all their packets in flight
// ---------------------------------------------------------------------------
template <int PF, int R>
__global__ __launch_bounds__(256) void w2_b1_kernel(WMat w2, int rows, int r,
                                                    const float *__restrict__ hid,
                                                    const float *__restrict__ b2, float t,
                                                    const float *__restrict__ tvec, int kd,
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
            raw[q][u] = (row0 + q < rows && row0 + q >= kd && p < NP)
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
                    raw[q][u] = (row0 + q < rows && row0 + q >= kd && p < NP)
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
        const int row = row0 + q;
        const float v = wave_sum(acc[q][0]) * row_scale<PF>(w2, row < rows ? row : 0);
        if (lane == 0 && row < rows) {
            const bool pre = row < kd;  // always-active prefix
            const float l = pre ? __builtin_inff() : v + b2[row];
            if (logits) logits[row] = l;
            mask[row] = (uint8_t)(pre || l > (tvec ? tvec[0] : t));
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
    bool silu;             // SwiGLU: SiLU instead of ReLU on the gate
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
                    v = gate_act(fmaf(vz, s, a.bias ? a.bias[i] : 0.0f), a.silu);
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

// Words per lane in the cross-wave reduction of the down projections: a lane
// parks its E column sums in a row of its own.  Rows of 32 words (4-bit
// packets) would all start on the same LDS bank, so every access of a wave
// would conflict 32 ways; one word of padding spreads them over the banks
// (175B-shaped 4-bit layer: 57.3 -> 56.4 us per layer).  Narrower rows keep
// the unpadded, vectorised layout, which measured as fast or faster.
template <int E> constexpr int red_pitch() { return E == 32 ? E + 1 : E; }

template <int FMT, int UR>
__global__ __launch_bounds__(256) void down_b1_kernel(DownB1Args a) {
    constexpr int E = PacketElems<FMT>::value;
    constexpr int RP = red_pitch<E>();
    __shared__ float red[64 * RP];
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
                float &rr = red[lane * RP + e];
                rr = (w == 0) ? acc[e] : rr + acc[e];
            }
        }
        __syncthreads();
    }
    const int col0 = slice * 64 * E;
    for (int t = threadIdx.x; t < 64 * E; t += blockDim.x)
        if (col0 + t < a.d) a.part[(size_t)c * a.d + col0 + t] = red[(t / E) * RP + t % E];
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
                                                            int32_t *total_out, int32_t *zero,
                                                            int n_zero, int zero_stride) {
    __shared__ float red[8][33];
    const int col = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int64_t e = (int64_t)blockIdx.x * 32 + col;
    float s = 0.0f;
    if (e < n) {
        constexpr int V = 16;
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
    // (each chunk counter is 64 bits: two words)
    if (blockIdx.x == 0)
        for (int k = threadIdx.x; k < n_zero; k += blockDim.x) {
            zero[(size_t)k * zero_stride] = 0;
            zero[(size_t)k * zero_stride + 1] = 0;
        }
}

// ---------------------------------------------------------------------------
// One layer of the single-token decode after predictor layer 1, in one
// launch: G row-group workgroups (predictor layer 2 + threshold + gate/up
// gather) followed by C*S down-projection workgroups (S column slices per
// chunk of NG consecutive row groups).
//
// Row group g owns the interleaved W2 rows {g + G*k : k < RB}, so the
// hot-first rows spread one per group.  It computes their logits in passes
// of one row per wave, writes the mask, keeps its active rows as a register
// mask (ascending within the group), computes the activation of each active
// row with all four waves sharing the row's packets (two rows at a time for
// most row kinds), and writes the RB slots [g*RB, g*RB + RB) of lst_i / lst_a
// (neuron, activation; its active rows first, the rest neuron -1).  It then
// publishes them: the slots are written with agent-scope (L2-coherent)
// stores, and once they have completed, done[c] of its chunk c = g / NG is
// incremented.
//
// A down-projection workgroup (chunk c, slice) waits until done[c] counts
// every group of its chunk, then reads the chunk's slots (contiguous, with
// agent-scope loads) and accumulates its column slice.  Its workgroup index is above every row
// group's, so every group it waits for was dispatched before it and never
// waits itself; the wait is also bounded, and a workgroup that runs out of
// patience writes NaN partial sums instead of hanging.  Chunks are ranges of
// consecutive groups, so the chunks of the first groups (which hold the
// hottest rows) are complete first and the down projection overlaps the
// tail of the gather.
// ---------------------------------------------------------------------------
// Chunk counters sit 4 KB apart: atomics and polls on one memory line
// serialise, and 64 counters packed into two lines cost tens of microseconds
// per layer.
constexpr int kDoneStride = kFusedDoneStride;

struct FusedArgs {
    WMat w2, wa, wu;
    int d, d_ffn, r;
    int groups;           // row groups of RB rows (rows interleaved with stride groups)
    const float *hid;     // [r]
    const float *b2;      // [d_ffn]
    float t;
    int kd;               // always-active prefix: rows [0, kd) are not scored
    bool silu;            // SwiGLU: SiLU instead of ReLU on the gate
    const float *bias;    // [d_ffn] or nullptr
    const float *h;       // [d] residual stream (un-normalised)
    const float *scale;   // device RMS scale
    float *logits;        // [d_ffn] or nullptr
    uint8_t *mask;        // [d_ffn]
    int32_t *lst_i;       // [G*RB]
    float *lst_a;         // [G*RB]
    int passes;           // W2 passes of 4 rows per row group (fused_passes)
    int per_chunk;        // NG: consecutive groups per down-projection chunk
    int32_t *done;        // [C * kDoneStride] per chunk, 64 bits: groups published (low
                          // word), groups with active rows (high word); zero at launch
    bool adapt;           // host only: the token's threshold is at scale[1], not t
};

// Row groups of the layer kernel.  A group's W2 rows are read in P passes of
// one row per wave (4 rows a pass; each pass's rows are requested once the
// previous pass's are multiplied), so a group costs the registers of one pass
// whatever its size.  P is chosen per layer (fused_passes) so that the layer
// has about kTargetGroups row groups -- four per CU of the 256 CUs: one round
// of resident workgroups (at five waves per SIMD with a slot per CU left to
// the down workgroups) --
// and a group at most 64 rows (its list slots are written by its first wave).
// Found by sweeping fixed group sizes per layer of a decode step (us), against
// the best one-pass groups: 175B-shaped 4-bit rows, 48 rows (12 passes) 52.1
// against 20 rows 56.4 (one-row passes for 40, 44, 56, 64 rows 54.0, 54.2,
// 53.4, 53.8; 48 rows in passes of 16, 12 or 8 rows 53.9, 53.2, 53.6);
// 40B-shaped ReLU, 32 rows (8 passes) 40.3 against 12 rows 41.4 (24 rows in
// passes of 12: 41.6; 32 rows in passes of 8: 40.4); 70B-shaped ReGLU, 28
// rows (7 passes) 46.1 against 8 rows 46.4 (12, 16, 24 and 32 rows 0.5-2.3%
// slower); 7B-shaped ReGLU, 12 rows (3 passes) 23.87 against 8 rows 23.87 (16
// and 28 rows slower).  The per-layer pass count against those fixed shapes
// per kind (whole decode steps on one box, ms): 70B 3.629 vs 3.681, 40B 2.333
// vs 2.336, 7B 0.781 vs 0.775, 175B 5.123 vs 5.099.
// (Other targets at the 70B shape, with paired gathers at four waves per SIMD:
// 896 groups of 32 rows 3.699 ms per step, 1152 of 24 rows 3.915, against 3.599.)
constexpr int kTargetGroups = 1024;
constexpr int kMaxGroupRows = 64;
// One row per wave in a pass.  (Small gated layers did better with 8-row
// groups in one pass of two rows per wave until their active rows were
// gathered in pairs; since then 12-row groups in three passes are faster at
// the 7B shape: 0.773 against 0.778 ms per step.)
constexpr int kPassRowsPerWave = 1;

template <int PF, int FMT, bool GATED, int UA, bool ADAPT>
__device__ __forceinline__ void fused_group(const FusedArgs &a, const int g) {
    constexpr int EP = PacketElems<PF>::value;
    constexpr int E = PacketElems<FMT>::value;
    constexpr int PL = PF == kFP8 ? 1 : 2;  // W2 packets per lane per row (one pass)
    constexpr int RW = kPassRowsPerWave;
    constexpr int RBP = 4 * RW;  // rows per pass
    __shared__ uint32_t s_bits[4];
    __shared__ float s_bias[kMaxGroupRows];  // bias of every row of the group, by local index
    __shared__ float s_part[kMaxGroupRows][4][2];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int G = a.groups;
    const int NPS = a.passes;  // W2 passes; row k = RBP ps + 4q + wv of the group in pass ps
    const int RB = RBP * NPS;  // rows per row group (one group per workgroup)
    const int NPr = a.r / EP, NPd = a.d / E;

    // One pass's W2 operands of this wave, straight into registers: the rows
    // g + G*(RBP ps + 4q + wv), q < RW, and their b2 entries and row scales
    // (lane q holds row q's).  Addresses are clamped into range and
    // out-of-range values discarded, so the loads carry no branches.  Rows of
    // the always-active prefix are not scored: their loads are redirected to
    // one fixed row (the last), so that no W2 row of the prefix is read from
    // memory while every load stays unconditional.
    uint4 rc[RW][PL];
    float b2v, rsv;
    auto load_pass = [&](const int ps) {
#pragma unroll
        for (int q = 0; q < RW; ++q) {
            const int row = g + G * (RBP * ps + 4 * q + wv);
            const bool rv = row < a.d_ffn && row >= a.kd;
            const int rr = rv ? row : a.d_ffn - 1;
#pragma unroll
            for (int u = 0; u < PL; ++u) {
                const int p = u * 64 + lane;
                const uint4 v = ld_stream(row_ptr<PF>(a.w2, rr, a.r) + (p < NPr ? p : NPr - 1));
                rc[q][u] = (rv && p < NPr) ? v : make_uint4(0, 0, 0, 0);
            }
        }
        const int row = g + G * (RBP * ps + 4 * (lane < RW ? lane : 0) + wv);
        const int rb = row < a.d_ffn ? row : a.d_ffn - 1;
        b2v = a.b2[rb];
        rsv = row_scale<PF>(a.w2, rb);  // 1 except for fp8 predictor rows
    };
    // Everything the first pass needs is requested up front: its W2 rows, the
    // hid values of the lane's two packets, and the bias of each of the
    // group's rows (into LDS).
    load_pass(0);
    float hv[PL][EP];
#pragma unroll
    for (int u = 0; u < PL; ++u) {
        const int p = u * 64 + lane;
        float unused;
        load_packet_x<PF>(a.hid, p < NPr ? p : NPr - 1, hv[u], unused);
    }
    if ((int)threadIdx.x < RB) {
        const int row = g + G * (int)threadIdx.x;
        s_bias[threadIdx.x] = (a.bias && row < a.d_ffn) ? a.bias[row] : 0.0f;
    }
    // The RMS scale, and the threshold: the layer's, a kernel argument, or
    // (ADAPT, a threshold per token) the one predictor layer 1 wrote beside
    // the scale.  The plain step keeps the argument: a mask that waits on a
    // loaded threshold costs about 1 us per launch.
    float s, thr;
    if constexpr (ADAPT) {
        const float2 st = *reinterpret_cast<const float2 *>(a.scale);
        s = st.x;
        thr = st.y;
    } else {
        s = *a.scale;
        thr = a.t;
    }

    // logits, threshold, mask; bit RW ps + q of `bits` is the wave's row q of
    // pass ps (kept in a register: an LDS write of each pass's bits in the
    // loop cost 1-2% per layer)
    uint32_t bits = 0;
    auto do_pass = [&](const int ps) {
#pragma unroll
        for (int q = 0; q < RW; ++q) {
            float acc = 0.0f;
#pragma unroll
            for (int u = 0; u < PL; ++u)
                if (u * 64 + lane < NPr) acc = packet_dot_reg<PF>(rc[q][u], 1.0f, hv[u], 0.0f, acc);
            const float rq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rsv), q));
            const float v = wave_sum(acc) * rq;
            const float bq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b2v), q));
            const int row = g + G * (RBP * ps + 4 * q + wv);
            bool m = false;
            if (row < a.d_ffn) {
                const bool pre = row < a.kd;  // always-active prefix
                const float l = pre ? __builtin_inff() : v + bq;
                m = pre || l > thr;
                if (lane == 0) {
                    if (a.logits) a.logits[row] = l;
                    a.mask[row] = (uint8_t)m;
                }
            }
            bits |= (uint32_t)m << (RW * ps + q);
        }
    };
    // the first pass in straight-line code (the only one at the smallest
    // shapes), the rest in a loop
    do_pass(0);
    for (int ps = 1; ps < NPS; ++ps) {
        load_pass(ps);
        do_pass(ps);
    }
    if (lane == 0) s_bits[wv] = bits;
    // the group's active rows as one mask over the local index
    // k = RBP ps + 4q + wv (ascending k is ascending row g + G*k), built by
    // every thread
    __syncthreads();
    unsigned long long act_mask = 0;
    {
        const uint32_t b0 = s_bits[0], b1 = s_bits[1], b2 = s_bits[2], b3 = s_bits[3];
        for (int j = 0; j < RW * NPS; ++j)  // j = RW ps + q: local rows 4j .. 4j + 3
            act_mask |= (unsigned long long)(((b0 >> j) & 1u) | (((b1 >> j) & 1u) << 1) |
                                             (((b2 >> j) & 1u) << 2) | (((b3 >> j) & 1u) << 3))
                        << (4 * j);
    }
    const int n_act = __popcll(act_mask);

    // activations of the listed rows: the four waves share each row, lane
    // (wv, lane) always takes packets wv*64 + lane + 256u, so its activation
    // values are loaded once, into registers, after the first row's weights
    // have been requested (a group without active rows never reads them)
    // Packets past the end of a row load a clamped (valid) packet and meet
    // zero activation values, so every load is unconditional.
    float xv[UA][E], xs[UA];
    unsigned long long pending = act_mask;
    // The group's active rows two at a time, both rows' loads in flight
    // together: non-gated fp16 32-row groups hold ~2.5 active rows at the 40B
    // shape (40.4 -> 39.4 us per layer); gated fp16 28-row groups ~2.8 at the
    // 70B shape and 4-bit 48-row groups ~2.5 at the 175B shape, whose kernels
    // then run at four waves per SIMD for the pair's registers (steps 3.622 ->
    // 3.599 ms and 5.121 -> 5.043 ms; 7B 0.790 -> 0.776; at five waves the
    // 4-bit pair spilled, 52.2 -> 62.2 us per layer).  Gated rows wider than
    // 8192 columns and gated 4-bit rows keep one row at a time.
    if constexpr ((FMT != kQ4 && (!GATED || UA <= 4)) || (FMT == kQ4 && !GATED && UA == 2)) {
        for (int k = 0; k < n_act; k += 2) {
            const int kl0 = __ffsll(pending) - 1;
            pending &= pending - 1;
            const bool two = k + 1 < n_act;  // the same in every thread
            int kl1 = kl0;
            if (two) {
                kl1 = __ffsll(pending) - 1;
                pending &= pending - 1;
            }
            const int i0 = g + G * kl0, i1 = g + G * kl1;
            uint4 ra[UA], rb[UA], ua[UA], ub[UA];
            float sa[UA], sb[UA], sua[UA], sub[UA];
#pragma unroll
            for (int u = 0; u < UA; ++u) {
                const int p = wv * 64 + lane + 256 * u;
                const int pc = p < NPd ? p : NPd - 1;
                ra[u] = ld_stream(row_ptr<FMT>(a.wa, i0, a.d) + pc);
                sa[u] = packet_scale<FMT>(a.wa, i0, a.d, pc);
                if constexpr (GATED) {
                    ua[u] = ld_stream(row_ptr<FMT>(a.wu, i0, a.d) + pc);
                    sua[u] = packet_scale<FMT>(a.wu, i0, a.d, pc);
                }
            }
            if (two) {
#pragma unroll
                for (int u = 0; u < UA; ++u) {
                    const int p = wv * 64 + lane + 256 * u;
                    const int pc = p < NPd ? p : NPd - 1;
                    rb[u] = ld_stream(row_ptr<FMT>(a.wa, i1, a.d) + pc);
                    sb[u] = packet_scale<FMT>(a.wa, i1, a.d, pc);
                    if constexpr (GATED) {
                        ub[u] = ld_stream(row_ptr<FMT>(a.wu, i1, a.d) + pc);
                        sub[u] = packet_scale<FMT>(a.wu, i1, a.d, pc);
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < UA; ++u) {
                    rb[u] = make_uint4(0, 0, 0, 0);
                    sb[u] = 0.0f;
                    ub[u] = make_uint4(0, 0, 0, 0);
                    sub[u] = 0.0f;
                }
            }
            if (k == 0) {
#pragma unroll
                for (int u = 0; u < UA; ++u) {
                    const int p = wv * 64 + lane + 256 * u;
                    load_packet_x<FMT>(a.h, p < NPd ? p : NPd - 1, xv[u], xs[u]);
                }
            }
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
            float za = 0.0f, zb = 0.0f, zua = 0.0f, zub = 0.0f;
#pragma unroll
            for (int u = 0; u < UA; ++u) {
                za = packet_dot_reg<FMT>(ra[u], sa[u], xv[u], xs[u], za);
                zb = packet_dot_reg<FMT>(rb[u], sb[u], xv[u], xs[u], zb);
                if constexpr (GATED) {
                    zua = packet_dot_reg<FMT>(ua[u], sua[u], xv[u], xs[u], zua);
                    zub = packet_dot_reg<FMT>(ub[u], sub[u], xv[u], xs[u], zub);
                }
            }
            za = wave_sum(za);
            zb = wave_sum(zb);
            if constexpr (GATED) {
                zua = wave_sum(zua);
                zub = wave_sum(zub);
            }
            if (lane == 0) {
                s_part[k][wv][0] = za;
                s_part[k][wv][1] = zua;
                if (two) {
                    s_part[k + 1][wv][0] = zb;
                    s_part[k + 1][wv][1] = zub;
                }
            }
        }
    } else {
        for (int k = 0; k < n_act; ++k) {
            const int kl = __ffsll(pending) - 1;  // local index of the k-th active row
            pending &= pending - 1;
            const int i = g + G * kl;
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
    }
    __syncthreads();
    // Publish.  The chunk's 64-bit counter gains 1 per group (low word) and,
    // for a group with active rows, that group's bit (bit 32 + its index in
    // the chunk): a group without active rows writes no list slots and does
    // not wait for any store, and the down projection reads only the slots of
    // flagged groups.  (n_act is the same in every thread.)
    unsigned long long *const cnt64 = reinterpret_cast<unsigned long long *>(
        a.done + (size_t)(g / a.per_chunk) * kDoneStride);
    if (n_act == 0) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(cnt64, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
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
            // local index of the k-th active row
            unsigned long long m = act_mask;
            for (int j = 0; j < k; ++j) m &= m - 1;
            const int kl = __ffsll(m) - 1;
            v = gate_act(fmaf(vz, s, s_bias[kl]), a.silu);
            if constexpr (GATED) v *= vu * s;
            row = g + G * kl;
        }
        // agent-scope stores: coherent across the chip's L2 caches by
        // themselves, so publishing needs no cache write-back
        __hip_atomic_store(a.lst_i + (size_t)g * RB + k, row, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.lst_a + (size_t)g * RB + k, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // publish the list: the slots were written by lanes of wave 0 only; that
    // wave waits until its stores have completed, then counts the group in
    // (a release fence would also write back the whole L2, which costs far
    // more than the wait when every group does it)
    if (wv == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_sched_barrier(0);
        if (lane == 0)
            __hip_atomic_fetch_add(cnt64, 1ull + (1ull << (32 + g % a.per_chunk)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// down projection of one chunk's lists, one column slice: every thread
// requests its share of the chunk's slots at once, the active ones
// (neuron >= 0) are compacted into LDS in slot order, and wave w then takes
// rows w, w + 4, w + 8, ... of that list.
// ---------------------------------------------------------------------------
struct DownListArgs {
    WMat wd;
    int d, d_ffn;
    const int32_t *lst_i;
    const float *lst_a;
    int G, RB;
    int chunks;
    int per_chunk;         // consecutive groups per chunk
    float *part;           // [chunks, d]
    int32_t *chunk_cnt;    // [chunks] rows listed per chunk, or nullptr
    int wait_polls;        // polls before giving up on a chunk
    int32_t *giveups;      // device count of workgroups that gave up waiting
};

constexpr int kDownListMaxSlots = 64 * 20;  // list slots of one chunk's groups

template <int FMT, int UR>
__device__ __forceinline__ void down_chunk(const DownListArgs &a, const int slice, const int c,
                                           const bool ready, const uint32_t gmask) {
    constexpr int E = PacketElems<FMT>::value;
    constexpr int SPT = kDownListMaxSlots / 256;  // slots per thread
    constexpr int RP = red_pitch<E>();
    // The chunk's compacted list (neurons, then activations) in one array,
    // which also holds the four waves' column sums at the end when they fit
    // (fp32 and fp16 packets: two barriers instead of a chain of four, the
    // same order of additions; 70B-shaped layer 46.7 -> 46.5 us, 7B-shaped
    // 24.2 -> 23.9 us); wider packets sum through `red`.
    constexpr bool WREG = 4 * 64 * E <= 2 * kDownListMaxSlots;
    __shared__ float red[WREG ? 1 : 64 * RP];
    __shared__ int s_list[2 * kDownListMaxSlots];
    int *const s_i = s_list;
    float *const s_a = reinterpret_cast<float *>(s_list + kDownListMaxSlots);
    __shared__ int s_wc[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int NP = a.d / E;
    const int p = slice * 64 + lane;
    const bool pv = p < NP;
    const int g0 = c * a.per_chunk;
    const int ng = min(a.per_chunk, a.G - g0);  // groups of this chunk, at most 32 (launcher)
    const int S = ng * a.RB;                     // slots of this chunk
    const size_t base = (size_t)g0 * a.RB;
    const int col0 = slice * 64 * E;
    if (!ready) {
        // the chunk's lists never arrived: poison the partial sums, list no
        // rows, and count the give-up in the workspace status word
        for (int t = threadIdx.x; t < 64 * E; t += blockDim.x)
            if (col0 + t < a.d) a.part[(size_t)c * a.d + col0 + t] = __builtin_nanf("");
        if (threadIdx.x == 0) {
            if (a.chunk_cnt && slice == 0) a.chunk_cnt[c] = 0;
            __hip_atomic_fetch_add(a.giveups, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    int vi[SPT];
    float va[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        // agent-scope loads: they see the row groups' agent-scope stores
        // only the slots of groups that flagged active rows were written
        const int sl = (int)threadIdx.x + 256 * u;
        const bool live = sl < S && ((gmask >> (sl / a.RB)) & 1u);
        vi[u] = live ? __hip_atomic_load(a.lst_i + base + sl, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : -1;
        va[u] = live ? __hip_atomic_load(a.lst_a + base + sl, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 0.0f;
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
    if constexpr (WREG) {
        // every wave parks its sums in a region of its own (the list's LDS,
        // free once all waves are past their loads), then the four regions
        // are added in wave order
        float *wr = reinterpret_cast<float *>(s_list);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) wr[(wv * 64 + lane) * E + e] = acc[e];
        __syncthreads();
        for (int t = threadIdx.x; t < 64 * E; t += blockDim.x)
            if (col0 + t < a.d)
                a.part[(size_t)c * a.d + col0 + t] =
                    ((wr[t] + wr[64 * E + t]) + wr[2 * 64 * E + t]) + wr[3 * 64 * E + t];
    } else {
        for (int w = 0; w < 4; ++w) {
            if (wv == w) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float &rr = red[lane * RP + e];
                    rr = (w == 0) ? acc[e] : rr + acc[e];
                }
            }
            __syncthreads();
        }
        for (int t = threadIdx.x; t < 64 * E; t += blockDim.x)
            if (col0 + t < a.d) a.part[(size_t)c * a.d + col0 + t] = red[(t / E) * RP + t % E];
    }
}

// Polls before a down-projection workgroup gives up on its chunk (each poll
// is an atomic read at agent scope plus a short sleep; the default is far
// beyond any layer's run time).  Process-wide, read when a launch is enqueued.
static std::atomic<int> g_chunk_wait_polls{kChunkWaitPollsDefault};

void set_chunk_wait_polls(int polls) { g_chunk_wait_polls.store(polls); }

// Five resident waves per SIMD where the registers allow it without spills;
// gated fp16 / fp32 rows of 4097-8192 columns and non-gated 4-bit rows four
// (their pairs of gathered rows need 105-108 VGPRs; with about 1024 row
// groups, four per CU, they still fit one round); wider rows and gated 4-bit
// rows keep the compiler's own budget.
template <int FMT, bool GATED, int UA>
constexpr int layer_b1_waves() {
    return (FMT != kQ4 && GATED && UA == 4) || (FMT == kQ4 && !GATED && UA == 2) ? 4 : (FMT != kQ4 && UA <= 4) ? 5 : 1;
}

template <int PF, int FMT, bool GATED, int UA, int UR, bool ADAPT>
__global__ __launch_bounds__(256, (layer_b1_waves<FMT, GATED, UA>())) void layer_b1_kernel(
    FusedArgs f, DownListArgs dn, int slices) {
    if ((int)blockIdx.x < f.groups) {
        fused_group<PF, FMT, GATED, UA, ADAPT>(f, blockIdx.x);
        return;
    }
    const int q = (int)blockIdx.x - f.groups;
    const int c = q / slices, slice = q - c * slices;
    const int need = min(dn.per_chunk, dn.G - c * dn.per_chunk);
    __shared__ int s_ready;
    __shared__ uint32_t s_gmask;
    if (threadIdx.x == 0) {
        const unsigned long long *cnt64 =
            reinterpret_cast<const unsigned long long *>(f.done + (size_t)c * kDoneStride);
        int ok = 0;
        uint32_t gm = 0;
        for (int it = 0; it < dn.wait_polls; ++it) {
            const unsigned long long v =
                __hip_atomic_load(cnt64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((int)(uint32_t)v >= need) {
                ok = 1;
                gm = (uint32_t)(v >> 32);  // groups of the chunk with active rows
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        s_ready = ok;
        s_gmask = gm;
    }
    // every wave issues its slot loads after this barrier, so after the count
    // was seen complete.  The poll is relaxed on purpose: the slots are read
    // with agent-scope loads, which see the writers' agent-scope stores once
    // those have completed (each writer waits for that before its increment);
    // an acquire fence here invalidates the cache once per workgroup and
    // measured 45.5 against 38.6 us per launch at the 70B shape.
    __syncthreads();
    down_chunk<FMT, UR>(dn, slice, c, s_ready != 0, s_gmask);
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

// Packets per thread per pass: as many as one pass needs (a row of NP packets
// over 256 threads), at most 32 activation values per thread (4 packets for
// fp32 rows).
template <int PF, int RB, int UBMAX>
static void launch_w1x(const Layer &L, const float *h, float eps, bool normalize, float *hid,
                       float *scale_out, hipStream_t s, const float *tvec) {
    const spffn_layer_desc &D = L.desc;
    const int blocks = (D.r + RB - 1) / RB;
    const int NP = D.d / PacketElems<PF>::value;
    const int ub = NP <= 256 ? 1 : NP <= 512 ? 2 : 4;
    if (ub == 1 || UBMAX == 1)
        w1x_b1_kernel<PF, RB, 1><<<blocks, 256, 0, s>>>(L.w1, D.r, D.d, h, eps, normalize, D.p_b1,
                                                        hid, scale_out, tvec, L.t);
    else if (ub == 2 || UBMAX == 2)
        w1x_b1_kernel<PF, RB, (UBMAX < 2 ? UBMAX : 2)><<<blocks, 256, 0, s>>>(
            L.w1, D.r, D.d, h, eps, normalize, D.p_b1, hid, scale_out, tvec, L.t);
    else
        w1x_b1_kernel<PF, RB, UBMAX><<<blocks, 256, 0, s>>>(L.w1, D.r, D.d, h, eps, normalize,
                                                            D.p_b1, hid, scale_out, tvec, L.t);
}

hipError_t launch_w1_b1(const Layer &L, const float *h, float eps, bool normalize, float *hid,
                        float *scale_out, hipStream_t s, const float *tvec) {
    constexpr int RB = 4;
    // fp16 rows of at most 512 packets (two per thread): two rows per block,
    // twice the blocks (7B shape, d = 4096: 0.775 -> 0.767 ms per step; at
    // d = 8192 four rows per block stay ahead, 1.4525 against 1.4555 ms for 32
    // layers of the 70B shape)
    if (L.desc.p_dtype == SPFFN_F16 && L.desc.d <= 512 * 8)
        launch_w1x<kF16, 2, 2>(L, h, eps, normalize, hid, scale_out, s, tvec);
    else if (L.desc.p_dtype == SPFFN_F16)
        launch_w1x<kF16, RB, 4>(L, h, eps, normalize, hid, scale_out, s, tvec);
    else if (L.desc.p_dtype == SPFFN_FP8_E4M3)
        launch_w1x<kFP8, RB, 2>(L, h, eps, normalize, hid, scale_out, s, tvec);
    else
        launch_w1x<kF32, RB, 4>(L, h, eps, normalize, hid, scale_out, s, tvec);
    return hipGetLastError();
}

hipError_t launch_w2_b1(const Layer &L, const float *hid, float *logits, uint8_t *mask,
                        const float *tvec, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    constexpr int R = 8;
    const int blocks = (D.d_ffn + 4 * R - 1) / (4 * R);
    const size_t lds = (size_t)D.r * 4;
    if (D.p_dtype == SPFFN_F16)
        w2_b1_kernel<kF16, R><<<blocks, 256, lds, s>>>(L.w2, D.d_ffn, D.r, hid, D.p_b2, L.t, tvec,
                                                       D.dense_prefix, logits, mask);
    else if (D.p_dtype == SPFFN_FP8_E4M3)
        w2_b1_kernel<kFP8, R><<<blocks, 256, lds, s>>>(L.w2, D.d_ffn, D.r, hid, D.p_b2, L.t, tvec,
                                                       D.dense_prefix, logits, mask);
    else
        w2_b1_kernel<kF32, R><<<blocks, 256, lds, s>>>(L.w2, D.d_ffn, D.r, hid, D.p_b2, L.t, tvec,
                                                       D.dense_prefix, logits, mask);
    return hipGetLastError();
}

constexpr int kUpB1MaxBlocks = 1024;

hipError_t launch_up_b1(const Layer &L, const float *h, const float *scale, const int32_t *idx,
                        const int32_t *count, float *act, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    UpB1Args a{};
    const bool gated = D.kind != SPFFN_RELU;
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
    a.silu = D.kind == SPFFN_SWIGLU;
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

// W2 passes of a layer's row groups (4 waves x kPassRowsPerWave rows each):
// about kTargetGroups groups, at least one pass, at most kMaxGroupRows rows.
int fused_passes(const Layer &L) {
    constexpr int rp = 4 * kPassRowsPerWave;
    const int p = (L.desc.d_ffn + rp * kTargetGroups / 2) / (rp * kTargetGroups);
    return p < 1 ? 1 : p > kMaxGroupRows / rp ? kMaxGroupRows / rp : p;
}
int fused_rows_per_group(const Layer &L) { return 4 * kPassRowsPerWave * fused_passes(L); }
int fused_groups(const Layer &L) {
    const int RB = fused_rows_per_group(L);
    return (L.desc.d_ffn + RB - 1) / RB;
}

// Down-projection chunks: ranges of NG consecutive row groups, NG <= 32 (one
// flag bit per group in the chunk counter; a chunk's slots fit the down
// workgroup's LDS list), at least 128 chunks when there are that many
// groups: smaller chunks complete sooner after their last group, more of them
// cost more partial sums.  Measured per step, 70B shape: 32 chunks 4.15 ms,
// 64 3.87, 96 3.86, 128 3.83, 192 4.00, 256 4.27; 7B: 64 0.810, 128 0.802,
// 192 0.827.  175B 4-bit, per layer on the stack calibrated layer by layer
// (5.3% active): 96 chunks 57.96 us, 128 57.21, 192 58.44 with 20-row groups;
// 64 chunks 54.2, 96 53.1, 128 51.9, 192 52.6 with 48-row groups.  40B ReLU
// with 32-row groups: 64 chunks 39.8, 96 39.5, 128 39.35, 192 41.0.
int fused_per_chunk(const Layer &L) {
    const int G = fused_groups(L);
    // at most 32 groups (one flag bit each in the counter) whose list slots
    // fit the down workgroup's LDS list
    const int ngmax = std::min(32, kDownListMaxSlots / fused_rows_per_group(L));
    const int cmin = 128;
    int c = (G + ngmax - 1) / ngmax;
    if (c < cmin) c = cmin;
    if (c > G) c = G;
    return (G + c - 1) / c;
}

int fused_chunks(const Layer &L) {
    const int NG = fused_per_chunk(L);
    return (fused_groups(L) + NG - 1) / NG;
}

size_t fused_list_slots(const Layer &L) {
    return (size_t)fused_groups(L) * fused_rows_per_group(L);
}

// Column slices of the down projection: 64 packets each.
static int down_slices(const Layer &L) {
    return (L.desc.d / packet_elems(L.desc.w_dtype) + 63) / 64;
}

// Activated-row packets per lane: one pass of 256*UA packets covers a row.
static int fused_ua(const Layer &L) {
    const int NPd = L.desc.d / packet_elems(L.desc.w_dtype);
    return NPd <= 512 ? 2 : NPd <= 1024 ? 4 : 8;
}

bool fused_fits(const Layer &L) {
    // a W2 row must fit one pass of 2 packets per lane (1 for fp8 rows), an
    // activated row one pass of 8 packets per lane
    const int pl = L.desc.p_dtype == SPFFN_FP8_E4M3 ? 1 : 2;
    return L.desc.r / packet_elems(L.desc.p_dtype) <= 64 * pl &&
           L.desc.d / packet_elems(L.desc.w_dtype) <= 256 * 8;
}

template <int PF, int FMT, bool GATED, int UA, bool ADAPT>
static void launch_layer_t(const FusedArgs &f, const DownListArgs &dn, int slices, int blocks,
                           hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    constexpr int UR = FMT == kQ4 ? 8 : 16;
    // with timing events the dispatch itself is timestamped (the events bracket
    // the kernel's execution, not its launch)
    if (e0 || e1)
        hipExtLaunchKernelGGL(layer_b1_kernel<PF, FMT, GATED, UA, UR, ADAPT>, dim3(blocks),
                              dim3(256), 0,
                              s, e0, e1, 0, f, dn, slices);
    else
        layer_b1_kernel<PF, FMT, GATED, UA, UR, ADAPT><<<blocks, 256, 0, s>>>(f, dn, slices);
}

template <int PF, int FMT, bool GATED>
static void launch_layer_rw(const FusedArgs &f, const DownListArgs &dn, int slices, int blocks,
                            int UA, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (f.adapt) {
        if (UA == 2) launch_layer_t<PF, FMT, GATED, 2, true>(f, dn, slices, blocks, s, e0, e1);
        else if (UA == 4) launch_layer_t<PF, FMT, GATED, 4, true>(f, dn, slices, blocks, s, e0, e1);
        else launch_layer_t<PF, FMT, GATED, 8, true>(f, dn, slices, blocks, s, e0, e1);
    } else {
        if (UA == 2) launch_layer_t<PF, FMT, GATED, 2, false>(f, dn, slices, blocks, s, e0, e1);
        else if (UA == 4) launch_layer_t<PF, FMT, GATED, 4, false>(f, dn, slices, blocks, s, e0, e1);
        else launch_layer_t<PF, FMT, GATED, 8, false>(f, dn, slices, blocks, s, e0, e1);
    }
}

template <int PF, int FMT>
static void launch_layer_kind(const FusedArgs &f, const DownListArgs &dn, bool gated, int slices,
                              int blocks, int UA, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (gated) launch_layer_rw<PF, FMT, true>(f, dn, slices, blocks, UA, s, e0, e1);
    else launch_layer_rw<PF, FMT, false>(f, dn, slices, blocks, UA, s, e0, e1);
}

hipError_t launch_layer_b1(const Layer &L, const float *hid, const float *h, const float *scale,
                           float *logits, uint8_t *mask, int32_t *lst_i, float *lst_a,
                           int32_t *done, float *part, int32_t *chunk_cnt, int32_t *giveups,
                           bool adapt, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    const spffn_layer_desc &D = L.desc;
    const bool gated = D.kind != SPFFN_RELU;
    const int G = fused_groups(L), UA = fused_ua(L), C = fused_chunks(L), NG = fused_per_chunk(L);
    const int slices = down_slices(L);
    FusedArgs f{};
    f.w2 = L.w2;
    f.wa = gated ? L.gate : L.up;
    f.wu = L.up;
    f.d = D.d;
    f.d_ffn = D.d_ffn;
    f.r = D.r;
    f.groups = G;
    f.hid = hid;
    f.b2 = D.p_b2;
    f.t = L.t;
    f.kd = D.dense_prefix;
    f.silu = D.kind == SPFFN_SWIGLU;
    f.adapt = adapt;
    f.bias = D.b_act;
    f.h = h;
    f.scale = scale;
    f.logits = logits;
    f.mask = mask;
    f.lst_i = lst_i;
    f.lst_a = lst_a;
    f.passes = fused_passes(L);
    f.per_chunk = NG;
    f.done = done;
    DownListArgs dn{};
    dn.wd = L.down;
    dn.d = D.d;
    dn.d_ffn = D.d_ffn;
    dn.lst_i = lst_i;
    dn.lst_a = lst_a;
    dn.G = G;
    dn.RB = fused_rows_per_group(L);
    dn.chunks = C;
    dn.per_chunk = NG;
    dn.part = part;
    dn.chunk_cnt = chunk_cnt;
    dn.wait_polls = g_chunk_wait_polls.load();
    dn.giveups = giveups;
    const int blocks = G + C * slices;
    if (D.p_dtype == SPFFN_F16) {
        if (D.w_dtype == SPFFN_F16)
            launch_layer_kind<kF16, kF16>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
        else if (D.w_dtype == SPFFN_F32)
            launch_layer_kind<kF16, kF32>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
        else
            launch_layer_kind<kF16, kQ4>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
    } else if (D.p_dtype == SPFFN_FP8_E4M3) {
        if (D.w_dtype == SPFFN_F16)
            launch_layer_kind<kFP8, kF16>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
        else if (D.w_dtype == SPFFN_F32)
            launch_layer_kind<kFP8, kF32>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
        else
            launch_layer_kind<kFP8, kQ4>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
    } else {
        if (D.w_dtype == SPFFN_F16)
            launch_layer_kind<kF32, kF16>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
        else if (D.w_dtype == SPFFN_F32)
            launch_layer_kind<kF32, kF32>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
        else
            launch_layer_kind<kF32, kQ4>(f, dn, gated, slices, blocks, UA, s, ev_start, ev_stop);
    }
    return hipGetLastError();
}

hipError_t launch_reduce_groups(const float *part, int chunks, int64_t n, const float *resid,
                                float *y, hipStream_t s, const int32_t *chunk_cnt,
                                int32_t *total_out, int32_t *zero, int n_zero,
                                int zero_stride) {
    reduce_groups_kernel<<<(int)((n + 31) / 32), 256, 0, s>>>(part, chunks, n, resid, y, chunk_cnt,
                                                              total_out, zero, n_zero, zero_stride);
    return hipGetLastError();
}

}  // namespace spffn
