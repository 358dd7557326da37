// Batched (2 <= B <= 16 tokens) kernels on the matrix cores, for fp16 weights.
//
// A batch of B tokens turns every matrix-vector product of the layer into a
// product with B columns.  Each weight byte is then used B times, which at
// B = 16 is more multiply-adds than the vector units finish in the time HBM
// delivers the bytes, so the products run on v_mfma_f32_16x16x32_f16:
//
//   * the weights are the A operand (16 rows x 32 columns of K per
//     instruction), loaded from HBM straight into registers -- a lane's 8
//     halves are 16 contiguous bytes of one row;
//   * the activations are the B operand, kept in fp32 precision by splitting
//     each value into two halves, x = hi + lo with hi = fp16(x) and
//     lo = fp16(x - hi) (the pair carries about 22 significant bits); for
//     B <= 8 the hi and lo parts of the B tokens share one instruction
//     (columns 0..7 and 8..15) and the two halves of the result are added,
//     for B > 8 they take one instruction each into the same accumulator;
//   * the producers of those halves store them already in the instruction's
//     B layout ("packed", bpack_index), so that one load instruction reads
//     1 KB of contiguous memory; in token-major order each instruction would
//     touch 16 separate 64-byte pieces, and every wave of every workgroup
//     reads the same few lines at the same time;
//   * accumulation is fp32 throughout.
//
// Operand layouts of the instruction (wave64), checked on the device:
//   A lane l: row l % 16, k = 8 (l / 16) + i;   B lane l: column l % 16,
//   k = 8 (l / 16) + i;   D lane l: rows 4 (l / 16) + i, column l % 16.
// In that layout a load instruction could give each row only 64 contiguous
// bytes (four lanes), which HBM serves poorly, so the weights are loaded
// row-contiguously (256 bytes of each of 4 rows per instruction) into a
// wave-private LDS tile and read back in the A layout.
//
// The down projection contracts over the gathered rows, which are not
// contiguous in memory, so its workgroups stage 32 gathered rows x 512
// columns in LDS and read the B operand out of LDS transposed; the
// activations (split the same way) are the A operand, tokens as rows.
#include "device.h"

namespace spffn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

// 16 bytes of activations (8 halves) from L2-resident memory.
__device__ __forceinline__ half8 ld_half8(const _Float16 *p) {
    return as_half8(*reinterpret_cast<const uint4 *>(p));
}

// Packed B operand of 16 columns and K rows (K a multiple of 128): per 128-row
// step and per 32-row instruction s, lane l = 16q + m holds column m, rows
// 32s + 8q .. +7, as 16 contiguous bytes; 2048 halves per step.  Column m is
// token m's hi half (or, for B <= 8, token m - 8's lo half when m >= 8).
constexpr int kPackStep = 2048;
__device__ __forceinline__ size_t bpack_index(int m, int k) {
    return ((size_t)((k >> 7) * 4 + ((k >> 5) & 3)) * 64 + ((k >> 3) & 3) * 16 + m) * 8 + (k & 7);
}

// Store value v of token b, row k: hi and lo halves, into p0 (and p1 for B > 8).
__device__ __forceinline__ void bpack_store(_Float16 *p0, _Float16 *p1, int B, int b, int k,
                                            float v) {
    const _Float16 h = (_Float16)v;
    const _Float16 l = (_Float16)(v - (float)h);
    p0[bpack_index(b, k)] = h;
    if (B > 8) p1[bpack_index(b, k)] = l;
    else p0[bpack_index(b + 8, k)] = l;
}

// ---------------------------------------------------------------------------
// x [B, K] fp32 -> (optionally RMS-normalised) n, and its hi/lo fp16 split
// in the packed B-operand layout (hi: 16 x K halves; lo: used for B > 8).
// Block (b, c) writes columns [c K/C, (c+1) K/C) of token b; with
// normalisation every block of a token first sums the token's squares in the
// same fixed order, so all of them use the same scale.
// ---------------------------------------------------------------------------
constexpr int kSplitChunks = 8;

__global__ __launch_bounds__(256) void split_act_kernel(const float *__restrict__ x, int K,
                                                        float eps, int normalize,
                                                        float *__restrict__ n_out,
                                                        _Float16 *__restrict__ hi,
                                                        _Float16 *__restrict__ lo) {
    __shared__ float red[4];
    const int b = blockIdx.x;
    const float *xb = x + (size_t)b * K;
    float s = 1.0f;
    if (normalize) {
        float ss = 0.0f;
        const float4 *x4 = reinterpret_cast<const float4 *>(xb);
        for (int k = threadIdx.x; k < K / 4; k += blockDim.x) {
            const float4 v = x4[k];
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
        }
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
        __syncthreads();
        const float tot = red[0] + red[1] + red[2] + red[3];
        s = 1.0f / sqrtf(tot / (float)K + eps);
    }
    const int per = K / gridDim.y;
    const int c0 = blockIdx.y * per;
    for (int k = c0 + threadIdx.x; k < c0 + per; k += blockDim.x) {
        const float v = xb[k] * s;
        if (n_out) n_out[(size_t)b * K + k] = v;
        bpack_store(hi, lo, gridDim.x, b, k, v);
    }
}

// ---------------------------------------------------------------------------
// Batched GEMV on the matrix cores: for a tile of 16 rows (a dense range, or
// entries j of an index list) and B tokens,
//     Z[row, b] = sum_k W[row, k] x[b, k]
// over the workgroup's K range (WV waves, each 128-column steps of it, see
// below; blockIdx.y picks the range when K is split across workgroups),
// reduced over the waves in a fixed order, then one of three epilogues.
// ---------------------------------------------------------------------------
enum { kEpiPartial = 0, kEpiMask = 1, kEpiAct = 2, kEpiCount = 3 };

struct BgArgs {
    const _Float16 *wa;  // [rows, K] (gate for ReGLU, else the one matrix)
    const _Float16 *wu;  // [rows, K] W_up for ReGLU
    int K;
    int rows;              // rows of the matrix
    const int32_t *idx;    // gathered: row of list entry j; nullptr: dense
    const int32_t *count;  // device count of the list (gathered only)
    // Gathered from tile masks instead (tmask != nullptr): bit r of tmask[t]
    // marks row 16t + r; list entry j is the j-th marked row in ascending
    // order.  The kernel then writes the list it used to idx_out and its
    // length to *count_out (and *count_out2 when given).
    const uint16_t *tmask;
    int ntiles;
    int32_t *idx_out, *count_out, *count_out2;
    const _Float16 *xhi, *xlo;  // packed B operand (bpack_index), 16 x K halves each
    int B;
    // epilogues
    const float *bias;     // [rows] or nullptr (mask: b2; act: b_act)
    float t;               // mask: logit threshold
    const float *tvec;     // mask: per-token thresholds [B] replacing t, or nullptr
    int kd;                // mask: rows [0, kd) always active (logit reported +inf)
    float *part;           // partial: [gridDim.y, B, rows]
    float *logits;         // mask: [B, rows] or nullptr
    uint8_t *mask;         // mask: [B, rows] or nullptr
    uint8_t *uni;          // mask: [rows] or nullptr
    uint16_t *tmask_out;   // mask: union bits of each 16-row tile, or nullptr
    _Float16 *ahi, *alo;   // act: [B, ld_act], entry j of the list
    int ld_act;
    const float *tsc;      // act: per-token scale of the products (raw input), or nullptr
    bool silu;             // act: SwiGLU (SiLU instead of ReLU on the gate)
    int32_t *counts;       // count: [rows] += tokens with Z + bias > 0
};

template <int WV, int T, bool GATED, bool SPLIT2, int EPI>
__global__ __launch_bounds__(64 * WV) void bgemv_kernel(BgArgs a) {
    constexpr int NM = GATED ? 2 : 1;
    // T tiles of 16 rows per workgroup; every wave runs all T tiles over its K
    // range, so each activation operand it loads feeds T tiles.
    // Per wave: the current 16 rows x 128 columns of each tile and matrix (16
    // chunks of 16 B per row, chunk c of row r at slot c ^ r); reused for the
    // cross-wave sums once the K loop is done.
    __shared__ uint4 stg[WV][NM][T][16][16];
    __shared__ uint32_t s_any[16 * T];
    __shared__ int s_rows[16 * T];
    __shared__ int s_wsum[WV];
    float(*red)[NM][T][256] = reinterpret_cast<float(*)[NM][T][256]>(&stg[0][0][0][0][0]);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int m = lane & 15, q = lane >> 4;
    // The workgroup's K range (blockIdx.y picks it when K is split) is taken
    // in steps of 128 columns per wave.  With two tiles (B > 8) the waves are
    // interleaved: step i of wave w is columns k0 + 128 (WV i), so at every
    // step the workgroup's waves read adjacent 256-byte pieces of each row
    // (1 KB contiguous at WV = 4); measured at the 70B shape, 8 layers: 186.3
    // -> 175.3 us per layer at B = 16, 177.6 -> 167.8 at B = 12.  With one
    // tile (B <= 8, 8 or 16 waves) each wave keeps a contiguous range, which
    // measured 1-1.5% faster there.
    constexpr int IW = SPLIT2 ? WV : 1;     // step stride, in 128-column steps
    const int Kw = a.K / (WV * gridDim.y);  // columns per wave
    const int k0 = SPLIT2 ? blockIdx.y * WV * Kw + wv * 128 : (blockIdx.y * WV + wv) * Kw;

    // Length of the list.  From tile masks (gate/up products only): thread i
    // owns tiles [i M, i M + M), whose marked rows take the ranks
    // [base, base + own) of the list.
    const bool from_tiles = EPI == kEpiAct && a.tmask;
    int n_items, M = 0, own = 0, base = 0;
    if (from_tiles) {
        M = (a.ntiles + 64 * WV - 1) / (64 * WV);
        for (int u = 0; u < M; ++u) {
            const int t = (int)threadIdx.x * M + u;
            if (t < a.ntiles) own += __popc((uint32_t)a.tmask[t]);
        }
        int incl = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) s_wsum[wv] = incl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < WV; ++w) {
            const int v = s_wsum[w];
            before += w < wv ? v : 0;
            total += v;
        }
        base = before + incl - own;
        n_items = total;
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
            *a.count_out = total;
            if (a.count_out2) *a.count_out2 = total;
        }
    } else {
        n_items = a.idx ? min(max(*a.count, 0), a.rows) : a.rows;
    }

    // The grid may be smaller than the list (it is sized before the list is
    // known): workgroups loop over row tiles.
    for (int j0 = blockIdx.x * 16 * T; j0 < n_items; j0 += gridDim.x * 16 * T) {
        if (from_tiles) {
            // rows of list entries [j0, j0 + 16T), by the threads whose ranks cover them
            const int lim = j0 + 16 * T;
            if (own > 0 && base < lim && base + own > j0) {
                int rank = base;
                for (int u = 0; u < M && rank < lim; ++u) {
                    const int t = (int)threadIdx.x * M + u;
                    if (t >= a.ntiles) break;
                    uint32_t mk = a.tmask[t];
                    const int pop = __popc(mk);
                    if (rank + pop <= j0) {
                        rank += pop;
                        continue;
                    }
                    while (mk) {
                        const int b = __ffs(mk) - 1;
                        mk &= mk - 1;
                        if (rank >= j0 && rank < lim) s_rows[rank - j0] = 16 * t + b;
                        ++rank;
                    }
                }
            }
            __syncthreads();
        }
        auto row_of = [&](int j) { return from_tiles ? s_rows[j - j0] : (a.idx ? a.idx[j] : j); };
        // Weight loads are row-contiguous: load g (of 4) gives lane l chunk l & 15
        // (8 columns) of tile row 4g + (l >> 4), i.e. 256 contiguous bytes of each
        // of 4 rows per instruction.  Through LDS each lane then picks up the
        // chunks of the A layout (row m, columns 32s + 8q).
        const _Float16 *pa[T][4], *pu[T][4];
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int jr = j0 + 16 * t + 4 * g + (lane >> 4);
                int rr = row_of(jr < n_items ? jr : j0);
                rr = min(max(rr, 0), a.rows - 1);
                pa[t][g] = a.wa + (size_t)rr * a.K + k0 + 8 * (lane & 15);
                pu[t][g] = GATED ? a.wu + (size_t)rr * a.K + k0 + 8 * (lane & 15) : nullptr;
            }
        // B operand of this lane (packed): token m (SPLIT2), or token m & 7 of the
        // hi (m < 8) / lo (m >= 8) half, from the wave's first 128-row step on
        const int tok = SPLIT2 ? m : (m & 7);
        const bool tv = tok < a.B;
        const _Float16 *px = a.xhi + (size_t)(k0 >> 7) * kPackStep + 8 * lane;
        const _Float16 *pxl = a.xlo + (size_t)(k0 >> 7) * kPackStep + 8 * lane;

        f32x4 ca[T], cu[T];
#pragma unroll
        for (int t = 0; t < T; ++t) ca[t] = cu[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int kb = 0; kb < Kw; kb += 128) {
            uint4 ga[T][4], gu[T][4];
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    ga[t][g] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                   reinterpret_cast<const u32x4_t *>(pa[t][g] + kb * IW)));
                    if constexpr (GATED)
                        gu[t][g] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                       reinterpret_cast<const u32x4_t *>(pu[t][g] + kb * IW)));
                }
            half8 xb[4], xl[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const size_t o = (size_t)(kb >> 7) * IW * kPackStep + 512 * s;
                xb[s] = tv ? ld_half8(px + o) : zero8;
                if constexpr (SPLIT2) xl[s] = tv ? ld_half8(pxl + o) : zero8;
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r = 4 * g + (lane >> 4), c = (lane & 15) ^ r;
                    stg[wv][0][t][r][c] = ga[t][g];
                    if constexpr (GATED) stg[wv][NM - 1][t][r][c] = gu[t][g];
                }
            // the wave's own LDS writes are complete before any lane reads them
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int c = (4 * s + q) ^ m;
                    const half8 wa_ = as_half8(stg[wv][0][t][m][c]);
                    ca[t] = mfma16x16x32(wa_, xb[s], ca[t]);
                    if constexpr (SPLIT2) ca[t] = mfma16x16x32(wa_, xl[s], ca[t]);
                    if constexpr (GATED) {
                        const half8 wu_ = as_half8(stg[wv][NM - 1][t][m][c]);
                        cu[t] = mfma16x16x32(wu_, xb[s], cu[t]);
                        if constexpr (SPLIT2) cu[t] = mfma16x16x32(wu_, xl[s], cu[t]);
                    }
                }
            // and all reads are done before the next step overwrites the slots
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        __syncthreads();  // every wave is done with its slots before they hold sums

        // fixed-order sum over the waves: red[w][.][t][r*16 + n]
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[wv][0][t][(4 * q + i) * 16 + m] = ca[t][i];
                if constexpr (GATED) red[wv][NM - 1][t][(4 * q + i) * 16 + m] = cu[t][i];
            }
        if (threadIdx.x < 16 * T) s_any[threadIdx.x] = 0u;
        __syncthreads();
        // entry e < 256 T is (tile t = e / 256, row r = e / 16 % 16, column n =
        // e % 16); for B <= 8 the entries n < 8 add the lo half held in column n + 8
        for (int e = threadIdx.x; e < 256 * T; e += blockDim.x) {
            const int t = e >> 8, te = e & 255, r = te >> 4, n = te & 15;
            if (n >= a.B || (!SPLIT2 && n >= 8)) continue;
            float za = 0.0f, zu = 0.0f;
            for (int w = 0; w < WV; ++w) {
                za += red[w][0][t][te];
                if (!SPLIT2) za += red[w][0][t][te + 8];
                if constexpr (GATED) {
                    zu += red[w][NM - 1][t][te];
                    if (!SPLIT2) zu += red[w][NM - 1][t][te + 8];
                }
            }
            const int jj = j0 + 16 * t + r;
            if (jj >= n_items) continue;
            const int rr = row_of(jj);
            if (from_tiles && n == 0) a.idx_out[jj] = rr;
            if constexpr (EPI == kEpiPartial) {
                a.part[((size_t)blockIdx.y * a.B + n) * a.rows + rr] = za;
            } else if constexpr (EPI == kEpiMask) {
                const bool pre = rr < a.kd;
                const float l = pre ? __builtin_inff() : za + (a.bias ? a.bias[rr] : 0.0f);
                const bool mk = pre || l > (a.tvec ? a.tvec[n] : a.t);
                if (a.logits) a.logits[(size_t)n * a.rows + rr] = l;
                if (a.mask) a.mask[(size_t)n * a.rows + rr] = (uint8_t)mk;
                if (mk) atomicOr(&s_any[16 * t + r], 1u);  // LDS
            } else if constexpr (EPI == kEpiCount) {
                if (za + (a.bias ? a.bias[rr] : 0.0f) > 0.0f) atomicAdd(&s_any[16 * t + r], 1u);
            } else {
                const float sc = a.tsc ? a.tsc[n] : 1.0f;
                float v = gate_act(fmaf(za, sc, a.bias ? a.bias[rr] : 0.0f), a.silu);
                if constexpr (GATED) v *= zu * sc;
                const _Float16 h = (_Float16)v;
                a.ahi[(size_t)n * a.ld_act + jj] = h;
                a.alo[(size_t)n * a.ld_act + jj] = (_Float16)(v - (float)h);
            }
        }
        if constexpr (EPI == kEpiCount) {
            // one thread per row adds the tile's count (launches of one
            // profile call run in stream order, so plain updates suffice)
            __syncthreads();
            if ((int)threadIdx.x < 16 * T && j0 + (int)threadIdx.x < n_items)
                a.counts[row_of(j0 + threadIdx.x)] += (int32_t)s_any[threadIdx.x];
        }
        if constexpr (EPI == kEpiMask) {
            __syncthreads();
            if ((int)threadIdx.x < 16 * T && a.uni && j0 + (int)threadIdx.x < n_items) {
                const int jj = j0 + threadIdx.x;
                a.uni[row_of(jj)] = (uint8_t)(s_any[threadIdx.x] != 0u);
            }
            // dense rows only: tile t of the workgroup is rows 16 (j0/16 + t) + r
            if ((int)threadIdx.x < T && a.tmask_out && !a.idx &&
                j0 + 16 * (int)threadIdx.x < n_items) {
                uint32_t mk = 0;
                for (int r = 0; r < 16; ++r) {
                    const int jj = j0 + 16 * threadIdx.x + r;
                    if (jj < n_items && s_any[16 * threadIdx.x + r] != 0u) mk |= 1u << r;
                }
                a.tmask_out[(j0 >> 4) + threadIdx.x] = (uint16_t)mk;
            }
        }
        __syncthreads();  // LDS is reused by the next row tile
    }
}

// hid[b, i] = ReLU(s_b * (sum over the K splits of part) + b1[i]), fp32 and
// split (packed B operand of predictor layer 2); block (x, b) takes rows
// [256x, 256x + 256) of token b.  With ss (sums of x^2 over each 32-column
// group of token b, nss of them) the input was the raw residual stream and
// s_b = 1 / sqrt(mean(x^2) + eps) is its RMS scale (every block of the token
// sums the same values in the same order; block 0 stores it to tsc[b]);
// without it s_b = 1.
__global__ __launch_bounds__(256) void w1_finish_kernel(const float *__restrict__ part, int KS,
                                                        int B, int r, const float *__restrict__ b1,
                                                        const float *__restrict__ ss, int nss,
                                                        float inv_k, float eps,
                                                        float *__restrict__ hid,
                                                        _Float16 *__restrict__ hhi,
                                                        _Float16 *__restrict__ hlo,
                                                        float *__restrict__ tsc) {
    __shared__ float red[4];
    const int b = blockIdx.y;
    // The K-split partial sums are requested before the RMS sums are reduced
    // (independent loads, one round trip instead of two; 70B layer at B = 4
    // 100.7 -> 99.1 us, B = 16 173.3 -> 171.5, 40B at B = 8 113.6 -> 112.1).
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const size_t t = (size_t)b * r + i;
    constexpr int KMAX = 8;
    float pv[KMAX];
#pragma unroll
    for (int c = 0; c < KMAX; ++c) pv[c] = (i < r && c < KS) ? part[(size_t)c * B * r + t] : 0.0f;
    float s = 1.0f;
    if (ss) {
        float q = 0.0f;
        for (int k = threadIdx.x; k < nss; k += blockDim.x) q += ss[(size_t)b * nss + k];
        q = wave_sum(q);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = q;
        __syncthreads();
        s = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) * inv_k + eps);
        if (blockIdx.x == 0 && threadIdx.x == 0 && tsc) tsc[b] = s;
    }
    if (i < r) {
        float v = 0.0f;  // the splits in ascending order
#pragma unroll
        for (int c = 0; c < KMAX; ++c)
            if (c < KS) v += pv[c];
        for (int c = KMAX; c < KS; ++c) v += part[(size_t)c * B * r + t];
        v = fmaxf(fmaf(v, s, b1 ? b1[i] : 0.0f), 0.0f);
        hid[t] = v;
        bpack_store(hhi, hlo, B, b, i, v);
    }
}

// y = resid + sum_c part[c] over [B, d] (chunks may be 0), summed as
// reduce_groups_kernel does, and in the same pass the packed fp16 split of y
// (the next layer's B operand, not normalised) and the sum of y^2 over each
// 32-column group, ss[b * d/32 + g], from which that layer takes its RMS scale.
// One block per 32 consecutive elements of one token (d a multiple of 32).
__global__ __launch_bounds__(256) void reduce_split_kernel(const float *__restrict__ part,
                                                           int chunks, int B, int d,
                                                           const float *resid, float *y,
                                                           _Float16 *__restrict__ hi,
                                                           _Float16 *__restrict__ lo,
                                                           float *__restrict__ ss) {
    __shared__ float red[8][33];
    const int col = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int64_t n = (int64_t)B * d;
    const int64_t e = (int64_t)blockIdx.x * 32 + col;
    float acc = 0.0f;
    constexpr int V = 8;
    for (int c0 = g; c0 < chunks; c0 += 8 * V) {
        float v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int cc = c0 + 8 * u;
            v[u] = cc < chunks ? part[(int64_t)cc * n + e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < V; ++u) acc += v[u];
    }
    red[g][col] = acc;
    __syncthreads();
    if (g == 0) {
        float tot = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) tot += red[k][col];
        const float v = resid[e] + tot;
        y[e] = v;
        bpack_store(hi, lo, B, (int)(e / d), (int)(e % d), v);
        float q = v * v;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) q += __shfl_xor(q, o, 64);
        if (col == 0) ss[blockIdx.x] = q;
    }
}

// ---------------------------------------------------------------------------
// Down projection: part[c, b, col] = sum over list entries j of chunk c of
// act[b, j] * W_down_t[idx[j], col], for the block's 512 columns.  Chunk c is
// entries [c*per, (c+1)*per) with per = the list length over the chunks,
// rounded up to a multiple of 32 (from the device count, so every chunk has
// work whatever the list length).  Per step the block stages 32 gathered rows
// x 512 columns (fp16) in LDS, rows 2p and 2p + 1 interleaved column by column
// (one 32-bit word holds both), so that a lane's B operand -- 8 consecutive
// rows of one column -- is four 32-bit LDS reads; wave w owns columns
// w*128 .. w*128+127 (8 tiles of 16).  The weights of the next two steps and
// the row indices of the one after are in flight during the multiplies.
// ---------------------------------------------------------------------------
constexpr int kDownCols = 512;
constexpr int kDownPitch = kDownCols + 4;  // words per staged row pair

struct BdArgs {
    const _Float16 *wd;  // W_down_t [rows, d]
    int d, rows;
    const int32_t *idx, *count;  // list (nullptr idx: dense)
    const _Float16 *ahi, *alo;   // [B, ld_act]
    int ld_act, B;
    float *part;  // [gridDim.y, B, d]
};

// Interleave two rows' 8 halves: word e = (lo: a[e], hi: b[e]).
__device__ __forceinline__ void interleave_rows(uint4 ra, uint4 rb, uint4 &w0, uint4 &w1) {
    const uint32_t x[4] = {ra.x, ra.y, ra.z, ra.w}, y[4] = {rb.x, rb.y, rb.z, rb.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = (x[i] & 0xFFFFu) | (y[i] << 16);
        o[2 * i + 1] = (x[i] >> 16) | (y[i] & 0xFFFF0000u);
    }
    w0 = make_uint4(o[0], o[1], o[2], o[3]);
    w1 = make_uint4(o[4], o[5], o[6], o[7]);
}

template <bool SPLIT2>
__global__ __launch_bounds__(256) void bdown_kernel(BdArgs a) {
    __shared__ __align__(16) uint32_t tile[16 * kDownPitch];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int m = lane & 15, q = lane >> 4;
    const int slice = blockIdx.x, c = blockIdx.y;
    const int n_items = a.idx ? min(max(*a.count, 0), a.rows) : a.rows;
    const int per = ((n_items + gridDim.y - 1) / gridDim.y + 31) / 32 * 32;
    const int j0 = min(n_items, c * per), j1 = min(n_items, j0 + per);
    const int col0 = slice * kDownCols;

    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // A operand source: token m (SPLIT2) or token m & 7 of hi (m < 8) / lo
    const int tok = SPLIT2 ? m : (m & 7);
    const bool tv = tok < a.B;
    const _Float16 *pa = (SPLIT2 || m < 8 ? a.ahi : a.alo) + (size_t)(tv ? tok : 0) * a.ld_act;
    const _Float16 *pal = a.alo + (size_t)(tv ? tok : 0) * a.ld_act;
    // Thread t stages packet p = t & 63 (8 columns) of the step's row pairs
    // pr = (t >> 6) + 4u, u < 4: rows 2 pr and 2 pr + 1.
    const int p = threadIdx.x & 63, r0 = threadIdx.x >> 6;
    auto rows_of = [&](int kb, int (&rv)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int jj = kb + 2 * (r0 + 4 * (u >> 1)) + (u & 1);
            int row = jj < j1 ? (a.idx ? a.idx[jj] : jj) : -1;
            rv[u] = row < 0 ? -1 : min(row, a.rows - 1);
        }
    };
    auto load_w = [&](const int (&rv)[8], uint4 (&vv)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 w = __builtin_bit_cast(
                uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(
                           a.wd + (size_t)(rv[u] < 0 ? 0 : rv[u]) * a.d + col0 + 8 * p)));
            vv[u] = rv[u] >= 0 ? w : make_uint4(0, 0, 0, 0);
        }
    };
    // Two weight buffers alternate (a: steps j0, j0 + 64, ...; b: j0 + 32, ...):
    // while step kb is multiplied, the weights of kb + 32 (other buffer) and
    // kb + 64 (this buffer, refilled right after it is staged) are in flight,
    // and each buffer's row indices are read one of its steps ahead.
    int ra[8], rb[8];
    uint4 va[8], vb[8];
    rows_of(j0, ra);
    load_w(ra, va);
    rows_of(j0 + 32, rb);
    load_w(rb, vb);
    rows_of(j0 + 64, ra);
    rows_of(j0 + 96, rb);
    auto step = [&](int kb, uint4 (&v)[8], int (&rv)[8]) {
        __syncthreads();  // the previous step's reads of the tile are done
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint4 w0, w1;
            interleave_rows(v[2 * u], v[2 * u + 1], w0, w1);
            uint32_t *dst = &tile[(r0 + 4 * u) * kDownPitch + 8 * p];
            *reinterpret_cast<uint4 *>(dst) = w0;
            *reinterpret_cast<uint4 *>(dst + 4) = w1;
        }
        __syncthreads();
        load_w(rv, v);           // step kb + 64
        rows_of(kb + 128, rv);   // the buffer's step after that
        // A: act of list entries kb + 8q .. +7 (zero past j1)
        half8 av, avl;
        const int ja = kb + 8 * q;
        if (tv && ja + 8 <= j1) {
            av = ld_half8(pa + ja);
            if constexpr (SPLIT2) avl = ld_half8(pal + ja);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = tv && ja + i < j1;
                av[i] = ok ? pa[ja + i] : (_Float16)0;
                if constexpr (SPLIT2) avl[i] = ok ? pal[ja + i] : (_Float16)0;
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int cc = wv * 128 + t * 16 + m;  // column within the slice
            // rows 8q .. 8q+7 of column cc: row pairs 4q .. 4q+3
            uint4 bw;
            bw.x = tile[(4 * q + 0) * kDownPitch + cc];
            bw.y = tile[(4 * q + 1) * kDownPitch + cc];
            bw.z = tile[(4 * q + 2) * kDownPitch + cc];
            bw.w = tile[(4 * q + 3) * kDownPitch + cc];
            const half8 bv = as_half8(bw);
            acc[t] = mfma16x16x32(av, bv, acc[t]);
            if constexpr (SPLIT2) acc[t] = mfma16x16x32(avl, bv, acc[t]);
        }
    };
    for (int kb = j0; kb < j1; kb += 64) {
        step(kb, va, ra);
        if (kb + 32 < j1) step(kb + 32, vb, rb);
    }

    // D lane (m, q): tokens 4q + i, column m of the tile.  B <= 8: rows 8..15
    // hold the lo half of tokens 0..7, held by lanes q + 2.
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int col = col0 + wv * 128 + t * 16 + m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = acc[t][i];
            if constexpr (!SPLIT2) v += __shfl_down(v, 32, 64);
            const int b = 4 * q + i;
            const bool mine = SPLIT2 ? true : q < 2;
            if (mine && b < a.B && col < a.d) a.part[((size_t)c * a.B + b) * a.d + col] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
constexpr int kBgWaves = 4;
constexpr int kW1Splits = 8;  // K splits of predictor layer 1 (few rows, long K)
constexpr int kBdChunks = 32;
// The gathered gate/up products have one row tile per 16 listed rows and a
// long K, so each tile gets several waves, each a K range (half as many at
// B > 8).  Gate and up: 8 waves (4 measured 3.5-9% slower at the 70B and 7B
// shapes).  One matrix (ReLU): 8 waves; with the 40B-shaped stack's 40% union
// at B = 8 (~830 tiles) 16 waves per tile took 119.3 us per layer, 8 waves
// 114.0 and 4 waves 128.3 (16 had paid only while the union was ~200 tiles,
// fewer than the CUs).
constexpr int kGatherWaves = 8, kGatherWavesG = 8;
// workgroups of a gather whose list comes from tile masks (two per CU)
constexpr int kGatherMaxTiles = 512;

bool mfma_fits(const Layer &L, int B) {
    const spffn_layer_desc &D = L.desc;
    if (B < 2 || B > 16) return false;
    if (D.w_dtype != SPFFN_F16 || D.p_dtype != SPFFN_F16) return false;
    // every wave's K range is whole 128-column steps
    const int kstep = 128 * kBgWaves;
    return D.d % (kstep * kW1Splits) == 0 && D.r % kstep == 0 && D.d % kDownCols == 0 &&
           D.d % (128 * kGatherWaves) == 0;
}

int mfma_down_chunks() { return kBdChunks; }
int mfma_w1_splits() { return kW1Splits; }

hipError_t launch_reduce_split(const float *part, int chunks, int B, int d, const float *resid,
                               float *y, _Float16 *hi, _Float16 *lo, float *ss, hipStream_t s) {
    reduce_split_kernel<<<(int)((int64_t)B * d / 32), 256, 0, s>>>(part, chunks, B, d, resid, y, hi,
                                                                   lo, ss);
    return hipGetLastError();
}

hipError_t launch_split_act(const float *x, int B, int K, float eps, bool normalize, float *n_out,
                            _Float16 *hi, _Float16 *lo, hipStream_t s) {
    // K is a multiple of 4096 on this path, so the chunks are whole float4s
    split_act_kernel<<<dim3(B, kSplitChunks), 256, 0, s>>>(x, K, eps, normalize ? 1 : 0, n_out,
                                                           hi, lo);
    return hipGetLastError();
}

// Two 16-row tiles per workgroup for the gathered gate/up products when
// B > 8 (the activation operand then costs as many bytes as the weights, so
// sharing it halves that traffic); grid.x counts 16-row tiles and is rounded
// to the workgroup's tiles here.  The predictor products (K = r or a split of
// d, two steps per wave) keep one tile: more, lighter workgroups measured
// 174.4 -> 173.2 us per 70B layer at B = 16 and 167.6 -> 165.9 at B = 12.
// WV1 / WV2: waves per workgroup for B <= 8 / B > 8 (each wave a K range).
template <bool GATED, int EPI, int WV1, int WV2>
static void launch_bg(const BgArgs &a, dim3 grid, hipStream_t s) {
    if (a.B > 8 && EPI != kEpiAct) {
        bgemv_kernel<WV2, 1, GATED, true, EPI><<<grid, 64 * WV2, 0, s>>>(a);
    } else if (a.B > 8) {
        grid.x = (grid.x + 1) / 2;
        bgemv_kernel<WV2, 2, GATED, true, EPI><<<grid, 64 * WV2, 0, s>>>(a);
    } else {
        bgemv_kernel<WV1, 1, GATED, false, EPI><<<grid, 64 * WV1, 0, s>>>(a);
    }
}

// Activation profile of fp16 rows on the matrix cores: tokens in groups of
// 16, each split into packed fp16 halves (hi, lo: 16 * d halves each), then
// one dense pass of the activated matrix with the count epilogue.
bool mfma_profile_fits(const Layer &L) {
    return L.desc.w_dtype == SPFFN_F16 && L.desc.d % (128 * kBgWaves) == 0;
}

hipError_t launch_mfma_profile(const Layer &L, const float *x, int N, int32_t *counts,
                               _Float16 *hi, _Float16 *lo, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    for (int b0 = 0; b0 < N; b0 += 16) {
        const int nb = N - b0 < 16 ? N - b0 : 16;
        split_act_kernel<<<dim3(nb, kSplitChunks), 256, 0, s>>>(x + (size_t)b0 * D.d, D.d, 0.0f,
                                                                0, nullptr, hi, lo);
        BgArgs a{};
        a.wa = reinterpret_cast<const _Float16 *>((D.kind != SPFFN_RELU ? L.gate : L.up).data);
        a.K = D.d;
        a.rows = D.d_ffn;
        a.xhi = hi;
        a.xlo = lo;
        a.B = nb;
        a.bias = D.b_act;
        a.counts = counts;
        launch_bg<false, kEpiCount, kBgWaves, kBgWaves>(a, dim3((D.d_ffn + 15) / 16, 1), s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_mfma_predict(const Layer &L, const _Float16 *xhi, const _Float16 *xlo, int B,
                               float *w1part, float *hid, _Float16 *hhi, _Float16 *hlo,
                               float *logits, uint8_t *mask, uint8_t *uni, uint16_t *tmask,
                               const float *ss, float eps, float *tsc, const float *tvec,
                               hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    BgArgs a{};
    a.wa = reinterpret_cast<const _Float16 *>(L.w1.data);
    a.K = D.d;
    a.rows = D.r;
    a.xhi = xhi;
    a.xlo = xlo;
    a.B = B;
    a.part = w1part;
    launch_bg<false, kEpiPartial, kBgWaves, kBgWaves>(a, dim3((D.r + 15) / 16, kW1Splits), s);
    w1_finish_kernel<<<dim3((D.r + 255) / 256, B), 256, 0, s>>>(
        w1part, kW1Splits, B, D.r, D.p_b1, ss, D.d / 32, 1.0f / (float)D.d, eps, hid, hhi, hlo, tsc);
    BgArgs b{};
    b.wa = reinterpret_cast<const _Float16 *>(L.w2.data);
    b.K = D.r;
    b.rows = D.d_ffn;
    b.xhi = hhi;
    b.xlo = hlo;
    b.B = B;
    b.bias = D.p_b2;
    b.t = L.t;
    b.tvec = tvec;
    b.kd = D.dense_prefix;
    b.logits = logits;
    b.mask = mask;
    b.uni = uni;
    b.tmask_out = tmask;
    launch_bg<false, kEpiMask, kBgWaves, kBgWaves>(b, dim3((D.d_ffn + 15) / 16, 1), s);
    return hipGetLastError();
}

// gate/up products over the list, then the down projection into part
static hipError_t mfma_ffn(const Layer &L, BgArgs a, dim3 grid, const int32_t *idx,
                           const int32_t *count, int B, float *part, hipStream_t s) {
    // a.tsc (if set) scales the products per token
    const spffn_layer_desc &D = L.desc;
    const bool gated = D.kind != SPFFN_RELU;
    a.wa = reinterpret_cast<const _Float16 *>((gated ? L.gate : L.up).data);
    a.wu = reinterpret_cast<const _Float16 *>(L.up.data);
    a.K = D.d;
    a.rows = D.d_ffn;
    a.B = B;
    a.bias = D.b_act;
    a.silu = D.kind == SPFFN_SWIGLU;
    if (gated) launch_bg<true, kEpiAct, kGatherWavesG, kGatherWavesG / 2>(a, grid, s);
    else launch_bg<false, kEpiAct, kGatherWaves, kGatherWaves / 2>(a, grid, s);

    BdArgs b{};
    b.wd = reinterpret_cast<const _Float16 *>(L.down.data);
    b.d = D.d;
    b.rows = D.d_ffn;
    b.idx = idx;
    b.count = count;
    b.ahi = a.ahi;
    b.alo = a.alo;
    b.ld_act = a.ld_act;
    b.B = B;
    b.part = part;
    const dim3 gd(D.d / kDownCols, kBdChunks);
    if (B > 8) bdown_kernel<true><<<gd, 256, 0, s>>>(b);
    else bdown_kernel<false><<<gd, 256, 0, s>>>(b);
    return hipGetLastError();
}

hipError_t launch_mfma_ffn(const Layer &L, const _Float16 *xhi, const _Float16 *xlo, int B,
                           const int32_t *idx, const int32_t *count, _Float16 *ahi, _Float16 *alo,
                           int ld_act, float *part, const float *tsc, hipStream_t s) {
    BgArgs a{};
    a.tsc = tsc;
    a.idx = idx;
    a.count = count;
    a.xhi = xhi;
    a.xlo = xlo;
    a.ahi = ahi;
    a.alo = alo;
    a.ld_act = ld_act;
    return mfma_ffn(L, a, dim3((L.desc.d_ffn + 15) / 16, 1), idx, count, B, part, s);
}

hipError_t launch_mfma_ffn_tiles(const Layer &L, const _Float16 *xhi, const _Float16 *xlo, int B,
                                 const uint16_t *tmask, int32_t *idx, int32_t *count,
                                 int32_t *count2, _Float16 *ahi, _Float16 *alo, int ld_act,
                                 float *part, const float *tsc, hipStream_t s) {
    BgArgs a{};
    a.tsc = tsc;
    a.tmask = tmask;
    a.ntiles = (L.desc.d_ffn + 15) / 16;
    a.idx_out = idx;
    a.count_out = count;
    a.count_out2 = count2;
    a.xhi = xhi;
    a.xlo = xlo;
    a.ahi = ahi;
    a.alo = alo;
    a.ld_act = ld_act;
    // at most one pass of resident workgroups; they loop over longer lists
    const int tiles = min(a.ntiles, kGatherMaxTiles * (B > 8 ? 2 : 1));
    return mfma_ffn(L, a, dim3(tiles, 1), idx, count, B, part, s);
}

}  // namespace spffn
