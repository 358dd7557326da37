// Internal declarations shared by the HIP sources of libspffn (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spffn.h"

namespace spffn {

constexpr int kWave = 64;

// Weight storage formats.  A "packet" is the 16 bytes one lane loads at a time:
// 4 fp32, 8 fp16, one 4-bit block of 32 codes (whose fp16 scale lives in a
// separate array), or 16 fp8 (E4M3) codes of a row with one fp32 scale.
enum Fmt : int { kF32 = 0, kF16 = 1, kQ4 = 2, kFP8 = 3 };

// One weight matrix [rows, cols] in device memory.
struct WMat {
    const uint8_t *data;     // fp32/fp16 elements, 4-bit or fp8 code region
    const uint16_t *scales;  // 4-bit only: fp16 scale bits [rows, cols/32]
    const float *rscale;     // fp8 only: one fp32 scale per row [rows]
    size_t stride;           // bytes from one row to the next (data region)
};

// Host-side layer handle (the C ABI's opaque spffn_layer).
struct Layer {
    spffn_layer_desc desc;
    float t;  // logit threshold ln(tau / (1 - tau)), binary64 rounded to binary32
    WMat gate, up, down, w1, w2;
};

// Workspace carve-up for a batch of B tokens.
struct WsLayout {
    size_t status;  // kWsStatusBytes at offset 0: int32 count of bounded waits that gave up
    size_t n, hid, mask, uni, idx, count, scale, act, gcnt, lst_i, lst_a, done, part, total;
    size_t xhi, xlo, hhi, hlo, ahi, alo, w1p;  // fp16 splits and partials of the batched path
    size_t tmask;                              // union bits per 16-row tile (batched path)
    size_t ss, tsc;  // batched decode: sums of squares of h per 32 columns, RMS scale per token
    int ld_act;  // row pitch (elements) of ahi / alo
    int chunks;  // neuron chunks of the down projection (partial-sum slots)
};

// Every workspace starts with a status block; its first int32 counts the
// down-projection workgroups whose bounded in-launch wait gave up.
constexpr size_t kWsStatusBytes = 256;

WsLayout layer_ws_layout(const Layer &L, int B);

// ---- launchers (each returns hipSuccess or the launch error) ---------------
hipError_t launch_threshold(const float *logits, int64_t n, float t, uint8_t *mask,
                            hipStream_t s);
hipError_t launch_compact(const uint8_t *mask, int n, int32_t *idx, int32_t *count,
                          hipStream_t s, int32_t *count2 = nullptr);
hipError_t launch_hot_first_order(const int32_t *counts, int n, int32_t *perm, hipStream_t s);
hipError_t launch_permute_rows(const void *src, void *dst, const int32_t *perm, int rows,
                               int64_t row_bytes, hipStream_t s);
hipError_t launch_q4_0_repack(const void *aos, void *soa, int rows, int cols, hipStream_t s);

// Dense row GEMVs of the predictor and the profile.
//   hid[b, j]   = max(W1[j] . x_b + b1[j], 0)
//   logits/mask = W2[i] . hid_b + b2[i] > t, union over b
//   counts[i]  += #{b : W[i] . x_b + bias[i] > 0}
hipError_t launch_gemv_hid(int fmt, WMat w, int rows, int cols, const float *x, int B,
                           const float *bias, float *out, hipStream_t s);
// tvec (or nullptr): per-token thresholds [B] replacing t
// kd: rows [0, kd) always active (an always-active prefix)
hipError_t launch_gemv_mask(int fmt, WMat w, int rows, int cols, const float *x, int B,
                            const float *bias, float t, const float *tvec, int kd,
                            float *logits, uint8_t *mask, uint8_t *uni, hipStream_t s);
hipError_t launch_gemv_count(int fmt, WMat w, int rows, int cols, const float *x, int B,
                             const float *bias, int32_t *counts, hipStream_t s);

// Gathered FFN.  idx == nullptr means every neuron (dense).
hipError_t launch_ffn_up(const Layer &L, const float *x, int B, const int32_t *idx,
                         const int32_t *count, float *act, hipStream_t s);
hipError_t launch_ffn_down(const Layer &L, int B, const int32_t *idx, const int32_t *count,
                           const float *act, float *part, int chunks, hipStream_t s);
// y[b, k] = sum_c part[c, b, k] (+ resid[b, k] when resid != nullptr)
hipError_t launch_reduce(const float *part, int chunks, int B, int d, const float *resid,
                         float *y, hipStream_t s);
hipError_t launch_rmsnorm(const float *h, int B, int d, float eps, float *n, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int32_t v, int n, hipStream_t s);
hipError_t launch_copy_words(const void *src, void *dst, int64_t n_words, hipStream_t s);
// measurement: read bytes (a multiple of 16) of buf once, folding into *sink
hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s);

int down_chunks(const Layer &L);
hipError_t launch_rms_scale(const float *h, int B, int d, float eps, float *scale, hipStream_t s);

// Single-token kernels (kernels_b1.hip); usable when b1_fits(L).
bool b1_fits(const Layer &L);
int down_b1_chunks(const Layer &L);
// scale_out (or nullptr): [0] the RMS scale, [1] the logit threshold (tvec[0]
// when tvec is given, else the layer's) for the single-token layer kernel
hipError_t launch_w1_b1(const Layer &L, const float *h, float eps, bool normalize, float *hid,
                        float *scale_out, hipStream_t s, const float *tvec = nullptr);
hipError_t launch_w2_b1(const Layer &L, const float *hid, float *logits, uint8_t *mask,
                        const float *tvec, hipStream_t s);
hipError_t launch_up_b1(const Layer &L, const float *h, const float *scale, const int32_t *idx,
                        const int32_t *count, float *act, hipStream_t s);
hipError_t launch_down_b1(const Layer &L, const int32_t *idx, const int32_t *count,
                          const float *act, float *part, int chunks, hipStream_t s);
// Batched path on the matrix cores (fp16 weights, 2 <= B <= 16).
bool mfma_fits(const Layer &L, int B);
// Activation profile (counts += tokens with a positive pre-activation) of
// fp16 rows on the matrix cores; hi, lo: 16 * d halves each of scratch.
bool mfma_profile_fits(const Layer &L);
hipError_t launch_mfma_profile(const Layer &L, const float *x, int N, int32_t *counts,
                               _Float16 *hi, _Float16 *lo, hipStream_t s);
int mfma_down_chunks();
int mfma_w1_splits();
hipError_t launch_split_act(const float *x, int B, int K, float eps, bool normalize, float *n_out,
                            _Float16 *hi, _Float16 *lo, hipStream_t s);
// tmask (or nullptr): the union bits of each 16-row tile, for launch_mfma_ffn_tiles.
// ss (or nullptr): the input is the raw residual stream, with its sums of
// squares per 32 columns (launch_reduce_split); the predictor then applies the
// RMS scale and stores it per token to tsc.
hipError_t launch_mfma_predict(const Layer &L, const _Float16 *xhi, const _Float16 *xlo, int B,
                               float *w1part, float *hid, _Float16 *hhi, _Float16 *hlo,
                               float *logits, uint8_t *mask, uint8_t *uni, uint16_t *tmask,
                               const float *ss, float eps, float *tsc, const float *tvec,
                               hipStream_t s);
// tsc (or nullptr): per-token scale of the products (the RMS scale of a raw input)
hipError_t launch_mfma_ffn(const Layer &L, const _Float16 *xhi, const _Float16 *xlo, int B,
                           const int32_t *idx, const int32_t *count, _Float16 *ahi, _Float16 *alo,
                           int ld_act, float *part, const float *tsc, hipStream_t s);
// The same over the union rows given by tile masks; the list is built on the
// device and written to idx[0..*count) (and *count2 when given).
hipError_t launch_mfma_ffn_tiles(const Layer &L, const _Float16 *xhi, const _Float16 *xlo, int B,
                                 const uint16_t *tmask, int32_t *idx, int32_t *count,
                                 int32_t *count2, _Float16 *ahi, _Float16 *alo, int ld_act,
                                 float *part, const float *tsc, hipStream_t s);
// y = resid + sum of chunks partial sums (chunks may be 0) over [B, d], plus the
// packed fp16 split of y and its sums of squares per 32 columns (ss: B * d/32)
hipError_t launch_reduce_split(const float *part, int chunks, int B, int d, const float *resid,
                               float *y, _Float16 *hi, _Float16 *lo, float *ss, hipStream_t s);

// y = resid + sum_c part[c]; optionally *total_out = sum of chunk_cnt[0..chunks)
// and zero[k * zero_stride + {0, 1}] = 0 for k < n_zero (64-bit counters)
hipError_t launch_reduce_groups(const float *part, int chunks, int64_t n, const float *resid,
                                float *y, hipStream_t s, const int32_t *chunk_cnt = nullptr,
                                int32_t *total_out = nullptr, int32_t *zero = nullptr,
                                int n_zero = 0, int zero_stride = 1);

// Fused predictor layer 2 + threshold + gate/up gather and its list-driven
// down projection (decode, one token).
bool fused_fits(const Layer &L);
int fused_groups(const Layer &L);
int fused_rows_per_group(const Layer &L);
int fused_chunks(const Layer &L);
int fused_per_chunk(const Layer &L);
size_t fused_list_slots(const Layer &L);  // list slots of the layer kernel (RB per row group)
// Predictor layer 2 + threshold + gate/up gather + down projection of one
// layer (single token) in one launch.  `scale` holds the RMS scale and the
// token's logit threshold, as launch_w1_b1 writes them; the threshold is read
// from there only with `adapt` (else the layer's own is used).  done holds fused_chunks(L) counters,
// kFusedDoneStride words apart, which must be zero (the whole region may be
// cleared).
constexpr int kFusedDoneStride = 1024;
// Bounded wait of the layer kernel's down-projection workgroups (polls).
constexpr int kChunkWaitPollsDefault = 1 << 18;
constexpr int kChunkWaitPollsMax = 1 << 24;
void set_chunk_wait_polls(int polls);
// giveups: device int32, incremented once per down-projection workgroup whose
// wait runs out (it then writes NaN partial sums and lists no rows).
hipError_t launch_layer_b1(const Layer &L, const float *hid, const float *h, const float *scale,
                           float *logits, uint8_t *mask, int32_t *lst_i, float *lst_a,
                           int32_t *done, float *part, int32_t *chunk_cnt, int32_t *giveups,
                           bool adapt, hipStream_t s, hipEvent_t ev_start = nullptr,
                           hipEvent_t ev_stop = nullptr);

}  // namespace spffn
