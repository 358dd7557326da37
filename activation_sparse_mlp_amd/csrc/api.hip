// C ABI of libspffn: argument validation, workspace layout and the launch
// sequences of predict / forward / decode_step.  Every entry point validates
// before it enqueues anything and never synchronises the host.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

using namespace spffn;

struct spffn_layer {
    Layer L;
};

struct spffn_model {
    std::vector<const spffn_layer *> layers;
    float eps;
    int d;
    bool uniform;  // every layer has the same shapes and storage types
};

namespace {

thread_local std::string g_err;

spffn_status fail(spffn_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

spffn_status hip_fail(hipError_t e, const char *what) {
    return fail(SPFFN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define SPFFN_HIP(call, what)                      \
    do {                                           \
        hipError_t e_ = (call);                    \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

int elems_multiple(int dtype) {
    return dtype == SPFFN_F32 ? 4 : dtype == SPFFN_F16 ? 8 : dtype == SPFFN_FP8_E4M3 ? 16 : 32;
}

WMat wmat(const void *p, int dtype, int rows, int cols) {
    WMat w{};
    w.data = static_cast<const uint8_t *>(p);
    w.scales = nullptr;
    w.rscale = nullptr;
    w.stride = dtype == SPFFN_F32 ? (size_t)cols * 4
               : dtype == SPFFN_F16 ? (size_t)cols * 2
               : dtype == SPFFN_FP8_E4M3 ? (size_t)cols
                                         : (size_t)cols / 2;
    if (dtype == SPFFN_Q4_0 && p)
        w.scales = reinterpret_cast<const uint16_t *>(w.data + (size_t)rows * (cols / 2));
    if (dtype == SPFFN_FP8_E4M3 && p)
        w.rscale = reinterpret_cast<const float *>(w.data + (size_t)rows * cols);
    return w;
}

struct Ws {
    int32_t *status;
    float *n, *hid, *act, *part, *scale, *lst_a, *w1p;
    uint8_t *mask, *uni;
    int32_t *idx, *count, *gcnt, *lst_i, *done;
    _Float16 *xhi, *xlo, *hhi, *hlo, *ahi, *alo;
    uint16_t *tmask;
    float *ss, *tsc;
    int ld_act;
    int chunks;
};

Ws carve(const Layer &L, int B, void *ws) {
    WsLayout lo = layer_ws_layout(L, B);
    uint8_t *base = static_cast<uint8_t *>(ws);
    Ws w;
    w.status = reinterpret_cast<int32_t *>(base + lo.status);
    w.n = reinterpret_cast<float *>(base + lo.n);
    w.hid = reinterpret_cast<float *>(base + lo.hid);
    w.mask = base + lo.mask;
    w.uni = base + lo.uni;
    w.idx = reinterpret_cast<int32_t *>(base + lo.idx);
    w.count = reinterpret_cast<int32_t *>(base + lo.count);
    w.scale = reinterpret_cast<float *>(base + lo.scale);
    w.act = reinterpret_cast<float *>(base + lo.act);
    w.gcnt = reinterpret_cast<int32_t *>(base + lo.gcnt);
    w.lst_i = reinterpret_cast<int32_t *>(base + lo.lst_i);
    w.lst_a = reinterpret_cast<float *>(base + lo.lst_a);
    w.done = reinterpret_cast<int32_t *>(base + lo.done);
    w.part = reinterpret_cast<float *>(base + lo.part);
    w.w1p = reinterpret_cast<float *>(base + lo.w1p);
    w.xhi = reinterpret_cast<_Float16 *>(base + lo.xhi);
    w.xlo = reinterpret_cast<_Float16 *>(base + lo.xlo);
    w.hhi = reinterpret_cast<_Float16 *>(base + lo.hhi);
    w.hlo = reinterpret_cast<_Float16 *>(base + lo.hlo);
    w.ahi = reinterpret_cast<_Float16 *>(base + lo.ahi);
    w.alo = reinterpret_cast<_Float16 *>(base + lo.alo);
    w.tmask = reinterpret_cast<uint16_t *>(base + lo.tmask);
    w.ss = reinterpret_cast<float *>(base + lo.ss);
    w.tsc = reinterpret_cast<float *>(base + lo.tsc);
    w.ld_act = lo.ld_act;
    w.chunks = lo.chunks;
    return w;
}

spffn_status check_batch(int32_t B) {
    if (B < 1 || B > SPFFN_MAX_BATCH)
        return fail(SPFFN_E_SHAPE, "batch B=%d outside [1, %d]", B, SPFFN_MAX_BATCH);
    return SPFFN_OK;
}

spffn_status check_ws(size_t need, const void *ws, size_t ws_bytes) {
    if (!ws) return fail(SPFFN_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(ws, 256)) return fail(SPFFN_E_ARG, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(SPFFN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return SPFFN_OK;
}

bool single(const Layer &L, int B) { return B == 1 && b1_fits(L); }

// The FFN part of one layer for B tokens over (idx, count) or every neuron.
// x is normalised by `scale` (device, per token) when scale != nullptr; the
// output is written to y, plus resid when resid != nullptr.
// split_ready: the batched path's fp16 split of x is already in w.xhi/xlo.
// tiles: (matrix-core path) the rows are the union rows marked in w.tmask
// instead of (idx, count); their list goes to w.idx / w.count (and count2).
// raw: the split in w.xhi/xlo is of the raw residual stream; the products are
// scaled by the RMS scale the predictor stored to w.tsc.  split_out: the
// reduce also writes the split of y and its sums of squares (w.ss) for the
// next layer.
spffn_status run_ffn(const Layer &L, const float *x, const float *scale, int B,
                     const int32_t *idx, const int32_t *count, const float *resid, float *y,
                     const Ws &w, hipStream_t s, bool split_ready = false, bool tiles = false,
                     int32_t *count2 = nullptr, bool raw = false, bool split_out = false) {
    if (single(L, B)) {
        SPFFN_HIP(launch_up_b1(L, x, scale, idx, count, w.act, s), "gather up/gate launch");
        SPFFN_HIP(launch_down_b1(L, idx, count, w.act, w.part, w.chunks, s), "gather down launch");
        SPFFN_HIP(launch_reduce_groups(w.part, w.chunks, L.desc.d, resid, y, s), "reduce launch");
        return SPFFN_OK;
    }
    // the batched kernels take an already normalised input (scale unused)
    if (mfma_fits(L, B)) {
        if (!split_ready)
            SPFFN_HIP(launch_split_act(x, B, L.desc.d, 0.0f, false, nullptr, w.xhi, w.xlo, s),
                      "split launch");
        const float *tsc = raw ? w.tsc : nullptr;
        if (tiles)
            SPFFN_HIP(launch_mfma_ffn_tiles(L, w.xhi, w.xlo, B, w.tmask, w.idx, w.count, count2,
                                            w.ahi, w.alo, w.ld_act, w.part, tsc, s),
                      "batched gather launch");
        else
            SPFFN_HIP(launch_mfma_ffn(L, w.xhi, w.xlo, B, idx, count, w.ahi, w.alo, w.ld_act,
                                      w.part, tsc, s),
                      "batched gather launch");
        if (split_out)
            SPFFN_HIP(launch_reduce_split(w.part, mfma_down_chunks(), B, L.desc.d, resid, y, w.xhi,
                                          w.xlo, w.ss, s),
                      "reduce launch");
        else
            SPFFN_HIP(launch_reduce_groups(w.part, mfma_down_chunks(), (int64_t)B * L.desc.d,
                                           resid, y, s),
                      "reduce launch");
        return SPFFN_OK;
    }
    SPFFN_HIP(launch_ffn_up(L, x, B, idx, count, w.act, s), "gather up/gate launch");
    SPFFN_HIP(launch_ffn_down(L, B, idx, count, w.act, w.part, w.chunks, s),
              "gather down launch");
    SPFFN_HIP(launch_reduce_groups(w.part, w.chunks, (int64_t)B * L.desc.d, resid, y, s),
              "reduce launch");
    return SPFFN_OK;
}

// Predictor of B tokens.  normalize: x is the residual stream and is RMS
// normalised first (decode); the RMS scale goes to w.scale.  tiles: the
// matrix-core path also writes the union bits per 16-row tile to w.tmask.
// raw: (matrix-core path) w.xhi/xlo hold the split of the raw residual
// stream and w.ss its sums of squares; the RMS scale is applied after layer
// 1 and stored per token to w.tsc.
spffn_status run_predict(const Layer &L, const float *x, int B, bool normalize, float eps,
                         float *logits, uint8_t *mask, uint8_t *uni, const Ws &w, hipStream_t s,
                         bool split_ready = false, bool tiles = false, bool raw = false,
                         const float *tvec = nullptr) {
    const spffn_layer_desc &D = L.desc;
    if (single(L, B)) {
        SPFFN_HIP(launch_w1_b1(L, x, eps, normalize, w.hid, w.scale, s), "predictor layer-1 launch");
        uint8_t *m = mask ? mask : uni;
        SPFFN_HIP(launch_w2_b1(L, w.hid, logits, m, tvec, s), "predictor layer-2 launch");
        if (mask && uni)
            SPFFN_HIP(hipMemcpyAsync(uni, mask, D.d_ffn, hipMemcpyDeviceToDevice, s), "union copy");
        return SPFFN_OK;
    }
    if (mfma_fits(L, B)) {
        if (!split_ready)
            SPFFN_HIP(launch_split_act(x, B, D.d, eps, normalize, w.n, w.xhi, w.xlo, s),
                      "split launch");
        SPFFN_HIP(launch_mfma_predict(L, w.xhi, w.xlo, B, w.w1p, w.hid, w.hhi, w.hlo, logits, mask,
                                      uni, tiles ? w.tmask : nullptr, raw ? w.ss : nullptr, eps,
                                      raw ? w.tsc : nullptr, tvec, s),
                  "batched predictor launch");
        return SPFFN_OK;
    }
    const float *xin = x;
    if (normalize) {
        SPFFN_HIP(launch_rmsnorm(x, B, D.d, eps, w.n, s), "rmsnorm launch");
        xin = w.n;
    }
    SPFFN_HIP(launch_gemv_hid(D.p_dtype, L.w1, D.r, D.d, xin, B, D.p_b1, w.hid, s),
              "predictor layer-1 launch");
    SPFFN_HIP(launch_gemv_mask(D.p_dtype, L.w2, D.d_ffn, D.r, w.hid, B, D.p_b2, L.t, tvec,
                               D.dense_prefix, logits, mask, uni, s),
              "predictor layer-2 launch");
    return SPFFN_OK;
}

}  // namespace

namespace spffn {

WsLayout layer_ws_layout(const Layer &L, int B) {
    const spffn_layer_desc &D = L.desc;
    WsLayout lo{};
    lo.chunks = down_chunks(L);
    lo.status = 0;
    size_t off = kWsStatusBytes;
    // The batched decode hands these from layer to layer, so they come first:
    // their offsets depend only on B and d, the same for every layer.
    const bool mf = B > 1 && mfma_fits(L, B);
    // packed B operands: 16 columns x K halves each (hi; lo for B > 8)
    const size_t nx = mf ? (size_t)16 * D.d * 2 : 0;
    lo.xhi = off;
    off += up256(nx);
    lo.xlo = off;
    off += up256(nx);
    lo.ss = off;
    off += up256(mf ? (size_t)B * (D.d / 32) * 4 : 0);
    lo.tsc = off;
    off += up256(mf ? (size_t)B * 4 : 0);
    lo.n = off;
    off += up256((size_t)B * D.d * 4);
    lo.hid = off;
    off += up256((size_t)B * D.r * 4);
    lo.mask = off;
    off += up256((size_t)B * D.d_ffn);
    lo.uni = off;
    off += up256((size_t)D.d_ffn);
    lo.idx = off;
    off += up256((size_t)D.d_ffn * 4);
    lo.count = off;
    off += 256;
    lo.scale = off;
    off += up256((size_t)B * 4);
    lo.act = off;
    off += up256((size_t)B * D.d_ffn * 4);
    const size_t G = (size_t)fused_groups(L), slots = fused_list_slots(L);
    lo.gcnt = off;  // rows listed per down-projection chunk (chunks <= G)
    off += up256(G * 4);
    lo.lst_i = off;
    off += up256(slots * 4);
    lo.lst_a = off;
    off += up256(slots * 4);
    lo.done = off;  // row groups published per down-projection chunk (single token)
    off += up256((size_t)fused_chunks(L) * kFusedDoneStride * 4);
    if (B == 1 && b1_fits(L)) {
        lo.chunks = down_b1_chunks(L);
        if (fused_fits(L) && fused_chunks(L) > lo.chunks) lo.chunks = fused_chunks(L);
    }
    if (B > 1 && mfma_fits(L, B) && mfma_down_chunks() > lo.chunks) lo.chunks = mfma_down_chunks();
    lo.part = off;
    off += up256((size_t)lo.chunks * B * D.d * 4);
    // fp16 splits of the batched path (only when it applies)
    lo.ld_act = (D.d_ffn + 7) / 8 * 8;
    const size_t nh = mf ? (size_t)16 * D.r * 2 : 0;
    const size_t na = mf ? (size_t)B * lo.ld_act * 2 : 0;
    lo.hhi = off;
    off += up256(nh);
    lo.hlo = off;
    off += up256(nh);
    lo.ahi = off;
    off += up256(na);
    lo.alo = off;
    off += up256(na);
    lo.w1p = off;
    off += up256(mf ? (size_t)mfma_w1_splits() * B * D.r * 4 : 0);
    lo.tmask = off;
    off += up256(mf ? (size_t)(D.d_ffn + 15) / 16 * 2 : 0);
    lo.total = off;
    return lo;
}

}  // namespace spffn

namespace {

// One-token decode through a uniform stack, three kernels per layer:
//   1. predictor layer 1, which also yields the RMS scale of h;
//   2. predictor layer 2 + threshold + gate/up gather + activation, with
//      per-group lists of the active neurons, and in the same launch the down
//      projection over those lists into per-chunk partial sums (each chunk
//      starts as soon as its groups have published their lists);
//   3. the fixed-order reduction of the partial sums with the residual add,
//      which also clears the chunk counters for the next layer.
spffn_status decode_one_token(const spffn_model *model, const float *x, float *h,
                              int32_t *layer_counts, const spffn_trace *trace, void *ws,
                              const float *tvec, hipStream_t s) {
    const int d = model->d;
    if (x != h) SPFFN_HIP(launch_copy_words(x, h, d, s), "input copy launch");
    {
        // the workspace comes uninitialised: clear the chunk counters once
        const Layer &L0 = model->layers[0]->L;
        SPFFN_HIP(launch_fill_i32(carve(L0, 1, ws).done, 0, fused_chunks(L0) * kFusedDoneStride, s),
                  "counter clear launch");
    }
    size_t mask_off = 0, logit_off = 0;
    for (size_t l = 0; l < model->layers.size(); ++l) {
        const Layer &L = model->layers[l]->L;
        const int F = L.desc.d_ffn;
        Ws w = carve(L, 1, ws);
        if (trace && trace->h_in)
            SPFFN_HIP(launch_copy_words(h, trace->h_in + l * (size_t)d, d, s), "trace copy launch");
        SPFFN_HIP(launch_w1_b1(L, h, model->eps, true, w.hid, w.scale, s, tvec ? tvec + l : nullptr),
                  "predictor layer-1 launch");
        float *lg = (trace && trace->logits) ? trace->logits + logit_off : nullptr;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (trace && trace->events) {
            e0 = (hipEvent_t)trace->events[2 * l];
            e1 = (hipEvent_t)trace->events[2 * l + 1];
        }
        const int chunks = fused_chunks(L);
        int32_t *lc = layer_counts ? layer_counts + l : nullptr;
        SPFFN_HIP(launch_layer_b1(L, w.hid, h, w.scale, lg, w.uni, w.lst_i, w.lst_a, w.done, w.part,
                                  lc ? w.gcnt : nullptr, w.status, tvec != nullptr, s, e0, e1),
                  "predictor layer-2 + gather + down launch");
        if (trace && trace->union_mask)
            SPFFN_HIP(hipMemcpyAsync(trace->union_mask + mask_off, w.uni, F, hipMemcpyDeviceToDevice,
                                     s),
                      "trace copy");
        // the reduce also clears the chunk counters for the next layer
        SPFFN_HIP(launch_reduce_groups(w.part, chunks, d, h, h, s, w.gcnt, lc, w.done, chunks,
                                       kFusedDoneStride),
                  "reduce launch");
        mask_off += F;
        logit_off += F;
    }
    return SPFFN_OK;
}

spffn_status check_decode(const spffn_model *model, const float *x, const float *h, int32_t B,
                          int32_t flags, const int32_t *layer_counts, const void *ws,
                          size_t ws_bytes);
spffn_status enqueue_decode(const spffn_model *model, const float *x, float *h, int32_t B,
                            int32_t flags, int32_t *layer_counts, const spffn_trace *trace,
                            void *ws, hipStream_t s, const float *tvec = nullptr);

}  // namespace

extern "C" {

const char *spffn_last_error(void) { return g_err.c_str(); }

const char *spffn_version(void) { return "spffn 0.1 (gfx950)"; }

spffn_status spffn_set_wait_limit(int32_t polls) {
    if (polls < 0 || polls > kChunkWaitPollsMax)
        return fail(SPFFN_E_ARG, "set_wait_limit: polls=%d outside [0, %d]", polls,
                    kChunkWaitPollsMax);
    set_chunk_wait_polls(polls);
    return SPFFN_OK;
}

spffn_status spffn_layer_create(const spffn_layer_desc *desc, spffn_layer **out) {
    if (!desc || !out) return fail(SPFFN_E_ARG, "layer_create: NULL desc or out");
    const spffn_layer_desc &D = *desc;
    if (D.d <= 0 || D.d_ffn <= 0 || D.r <= 0)
        return fail(SPFFN_E_SHAPE, "layer_create: d=%d d_ffn=%d r=%d must be positive", D.d,
                    D.d_ffn, D.r);
    if (D.kind != SPFFN_RELU && D.kind != SPFFN_REGLU && D.kind != SPFFN_SWIGLU)
        return fail(SPFFN_E_ARG, "layer_create: unknown kind %d", D.kind);
    if (D.w_dtype != SPFFN_F32 && D.w_dtype != SPFFN_F16 && D.w_dtype != SPFFN_Q4_0)
        return fail(SPFFN_E_DTYPE, "layer_create: unknown weight dtype %d", D.w_dtype);
    if (D.p_dtype != SPFFN_F32 && D.p_dtype != SPFFN_F16 && D.p_dtype != SPFFN_FP8_E4M3)
        return fail(SPFFN_E_DTYPE,
                    "layer_create: predictor dtype must be F32, F16 or FP8_E4M3, got %d",
                    D.p_dtype);
    if (D.d % elems_multiple(D.w_dtype))
        return fail(SPFFN_E_SHAPE, "layer_create: d=%d must be a multiple of %d for dtype %d", D.d,
                    elems_multiple(D.w_dtype), D.w_dtype);
    if (D.d % elems_multiple(D.p_dtype) || D.r % elems_multiple(D.p_dtype))
        return fail(SPFFN_E_SHAPE, "layer_create: d=%d and r=%d must be multiples of %d", D.d, D.r,
                    elems_multiple(D.p_dtype));
    if (!(D.tau > 0.0f && D.tau < 1.0f))
        return fail(SPFFN_E_ARG, "layer_create: tau=%g outside (0, 1)", (double)D.tau);
    if (D.dense_prefix < 0 || D.dense_prefix > D.d_ffn)
        return fail(SPFFN_E_SHAPE, "layer_create: dense_prefix=%d outside [0, d_ffn=%d]",
                    D.dense_prefix, D.d_ffn);
    if (!D.w_up || !D.w_down_t || !D.p_w1 || !D.p_b1 || !D.p_w2 || !D.p_b2)
        return fail(SPFFN_E_ARG, "layer_create: a required weight pointer is NULL");
    if (D.kind != SPFFN_RELU && !D.w_gate)
        return fail(SPFFN_E_ARG, "layer_create: a gated layer (ReGLU, SwiGLU) needs w_gate");
    const void *ptrs[] = {D.w_gate, D.w_up, D.w_down_t, D.p_w1, D.p_w2};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16))
            return fail(SPFFN_E_ARG, "layer_create: weight pointers must be 16-byte aligned");
    const void *fptrs[] = {D.b_act, D.p_b1, D.p_b2};
    for (const void *p : fptrs)
        if (p && !aligned(p, 4)) return fail(SPFFN_E_ARG, "layer_create: misaligned bias");

    spffn_layer *h = new (std::nothrow) spffn_layer;
    if (!h) return fail(SPFFN_E_ARG, "layer_create: out of host memory");
    h->L.desc = D;
    if (D.kind == SPFFN_RELU) h->L.desc.w_gate = nullptr;
    // threshold on the logit: sigmoid(l) > tau  <=>  l > ln(tau / (1 - tau))
    h->L.t = spffn_tau_threshold(D.tau);
    h->L.gate = wmat(h->L.desc.w_gate, D.w_dtype, D.d_ffn, D.d);
    h->L.up = wmat(D.w_up, D.w_dtype, D.d_ffn, D.d);
    h->L.down = wmat(D.w_down_t, D.w_dtype, D.d_ffn, D.d);
    h->L.w1 = wmat(D.p_w1, D.p_dtype, D.r, D.d);
    h->L.w2 = wmat(D.p_w2, D.p_dtype, D.d_ffn, D.r);
    *out = h;
    return SPFFN_OK;
}

void spffn_layer_destroy(spffn_layer *layer) { delete layer; }

float spffn_layer_threshold(const spffn_layer *layer) { return layer ? layer->L.t : NAN; }

spffn_status spffn_model_create(const spffn_layer *const *layers, int32_t n_layers,
                                float rms_eps, spffn_model **out) {
    if (!layers || !out || n_layers < 1)
        return fail(SPFFN_E_ARG, "model_create: need a non-empty layer array and out");
    if (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps))
        return fail(SPFFN_E_ARG, "model_create: rms_eps must be finite and >= 0");
    for (int i = 0; i < n_layers; ++i)
        if (!layers[i]) return fail(SPFFN_E_ARG, "model_create: layer %d is NULL", i);
    const int d = layers[0]->L.desc.d;
    for (int i = 1; i < n_layers; ++i)
        if (layers[i]->L.desc.d != d)
            return fail(SPFFN_E_SHAPE, "model_create: layer %d has d=%d, layer 0 has d=%d", i,
                        layers[i]->L.desc.d, d);
    spffn_model *m = new (std::nothrow) spffn_model;
    if (!m) return fail(SPFFN_E_ARG, "model_create: out of host memory");
    try {
        m->layers.assign(layers, layers + n_layers);
    } catch (...) {
        delete m;
        return fail(SPFFN_E_ARG, "model_create: out of host memory");
    }
    m->eps = rms_eps;
    m->d = d;
    m->uniform = true;
    for (int i = 1; i < n_layers; ++i) {
        const spffn_layer_desc &a = layers[0]->L.desc, &b = layers[i]->L.desc;
        if (a.d_ffn != b.d_ffn || a.r != b.r || a.kind != b.kind || a.w_dtype != b.w_dtype ||
            a.p_dtype != b.p_dtype)
            m->uniform = false;
    }
    *out = m;
    return SPFFN_OK;
}

void spffn_model_destroy(spffn_model *model) { delete model; }

size_t spffn_layer_workspace_bytes(const spffn_layer *layer, int32_t B) {
    if (!layer || B < 1 || B > SPFFN_MAX_BATCH) return 0;
    return layer_ws_layout(layer->L, B).total;
}

size_t spffn_model_workspace_bytes(const spffn_model *model, int32_t B) {
    if (!model || B < 1 || B > SPFFN_MAX_BATCH) return 0;
    size_t m = 0;
    for (const spffn_layer *l : model->layers) {
        const size_t v = layer_ws_layout(l->L, B).total;
        if (v > m) m = v;
    }
    return m;
}

spffn_status spffn_workspace_clear_status(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return fail(SPFFN_E_ARG, "workspace_clear_status: NULL workspace");
    if (!aligned(ws, 256)) return fail(SPFFN_E_ARG, "workspace must be 256-byte aligned");
    if (ws_bytes < kWsStatusBytes)
        return fail(SPFFN_E_WORKSPACE, "workspace has %zu bytes, less than its status block",
                    ws_bytes);
    SPFFN_HIP(launch_fill_i32(static_cast<int32_t *>(ws), 0, (int)(kWsStatusBytes / 4),
                              (hipStream_t)stream),
              "status clear launch");
    return SPFFN_OK;
}

spffn_status spffn_workspace_status(const void *ws, size_t ws_bytes, int32_t *giveups,
                                    void *stream) {
    if (!ws || !giveups) return fail(SPFFN_E_ARG, "workspace_status: NULL pointer");
    if (!aligned(ws, 256) || !aligned(giveups, 4))
        return fail(SPFFN_E_ARG, "workspace_status: misaligned workspace or output");
    if (ws_bytes < kWsStatusBytes)
        return fail(SPFFN_E_WORKSPACE, "workspace has %zu bytes, less than its status block",
                    ws_bytes);
    SPFFN_HIP(launch_copy_words(ws, giveups, 1, (hipStream_t)stream), "status copy launch");
    return SPFFN_OK;
}

spffn_status spffn_threshold(const float *logits, int64_t n, float t, uint8_t *mask,
                             void *stream) {
    if (!logits || !mask) return fail(SPFFN_E_ARG, "threshold: NULL pointer");
    if (n < 0) return fail(SPFFN_E_SHAPE, "threshold: n=%lld < 0", (long long)n);
    if (n == 0) return SPFFN_OK;
    SPFFN_HIP(launch_threshold(logits, n, t, mask, (hipStream_t)stream), "threshold launch");
    return SPFFN_OK;
}

spffn_status spffn_compact(const uint8_t *mask, int32_t n, int32_t *idx, int32_t *count,
                           void *stream) {
    if (!mask || !idx || !count) return fail(SPFFN_E_ARG, "compact: NULL pointer");
    if (n < 1) return fail(SPFFN_E_SHAPE, "compact: n=%d < 1", n);
    if (!aligned(idx, 4) || !aligned(count, 4))
        return fail(SPFFN_E_ARG, "compact: idx and count must be 4-byte aligned");
    SPFFN_HIP(launch_compact(mask, n, idx, count, (hipStream_t)stream), "compact launch");
    return SPFFN_OK;
}

spffn_status spffn_predict(const spffn_layer *layer, const float *x, int32_t B, float *logits,
                           uint8_t *mask, uint8_t *union_mask, void *ws, size_t ws_bytes,
                           void *stream) {
    if (!layer || !x) return fail(SPFFN_E_ARG, "predict: NULL layer or x");
    if (!logits && !mask && !union_mask)
        return fail(SPFFN_E_ARG, "predict: logits, mask and union_mask are all NULL");
    spffn_status st = check_batch(B);
    if (st) return st;
    if (!aligned(x, 16) || (logits && !aligned(logits, 4)))
        return fail(SPFFN_E_ARG, "predict: x must be 16-byte aligned, logits 4-byte");
    const Layer &L = layer->L;
    if ((st = check_ws(layer_ws_layout(L, B).total, ws, ws_bytes))) return st;
    Ws w = carve(L, B, ws);
    return run_predict(L, x, B, false, 0.0f, logits, mask, union_mask, w, (hipStream_t)stream);
}

spffn_status spffn_forward(const spffn_layer *layer, const float *x, int32_t B,
                           const uint8_t *mask, const int32_t *idx, const int32_t *count,
                           float *y, void *ws, size_t ws_bytes, void *stream) {
    if (!layer || !x || !y) return fail(SPFFN_E_ARG, "forward: NULL layer, x or y");
    spffn_status st = check_batch(B);
    if (st) return st;
    if (!aligned(x, 16) || !aligned(y, 16))
        return fail(SPFFN_E_ARG, "forward: x and y must be 16-byte aligned");
    if (!mask && (idx != nullptr) != (count != nullptr))
        return fail(SPFFN_E_ARG, "forward: idx and count must be given together");
    if (!mask && idx && (!aligned(idx, 4) || !aligned(count, 4)))
        return fail(SPFFN_E_ARG, "forward: misaligned idx or count");
    const Layer &L = layer->L;
    if ((st = check_ws(layer_ws_layout(L, B).total, ws, ws_bytes))) return st;
    Ws w = carve(L, B, ws);
    hipStream_t s = (hipStream_t)stream;
    const int32_t *use_idx = idx, *use_count = count;
    if (mask) {
        SPFFN_HIP(launch_compact(mask, L.desc.d_ffn, w.idx, w.count, s), "compact launch");
        use_idx = w.idx;
        use_count = w.count;
    }
    return run_ffn(L, x, nullptr, B, use_idx, use_count, nullptr, y, w, s);
}

spffn_status spffn_decode_step(const spffn_model *model, const float *x, float *h, int32_t B,
                               int32_t flags, int32_t *layer_counts, const spffn_trace *trace,
                               void *ws, size_t ws_bytes, void *stream) {
    spffn_status st = check_decode(model, x, h, B, flags, layer_counts, ws, ws_bytes);
    if (st) return st;
    return enqueue_decode(model, x, h, B, flags, layer_counts, trace, ws, (hipStream_t)stream);
}

float spffn_tau_threshold(float tau) {
    if (!(tau > 0.0f && tau < 1.0f)) return NAN;
    const double t = (double)tau;
    return (float)std::log(t / (1.0 - t));
}

spffn_status spffn_decode_step_adaptive(const spffn_model *model, const float *x, float *h,
                                        int32_t B, const float *thresholds,
                                        int32_t *layer_counts, const spffn_trace *trace,
                                        void *ws, size_t ws_bytes, void *stream) {
    if (!thresholds) return fail(SPFFN_E_ARG, "decode_step_adaptive: NULL thresholds");
    if (!aligned(thresholds, 4))
        return fail(SPFFN_E_ARG, "decode_step_adaptive: thresholds must be 4-byte aligned");
    spffn_status st = check_decode(model, x, h, B, 0, layer_counts, ws, ws_bytes);
    if (st) return st;
    return enqueue_decode(model, x, h, B, 0, layer_counts, trace, ws, (hipStream_t)stream,
                          thresholds);
}

struct spffn_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

spffn_status spffn_decode_graph_create(const spffn_model *model, const float *x, float *h,
                                       int32_t B, int32_t flags, int32_t *layer_counts, void *ws,
                                       size_t ws_bytes, spffn_graph **out) {
    if (!out) return fail(SPFFN_E_ARG, "decode_graph_create: NULL out");
    spffn_status st = check_decode(model, x, h, B, flags, layer_counts, ws, ws_bytes);
    if (st) return st;
    hipStream_t cs = nullptr;
    SPFFN_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "capture stream");
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return fail(SPFFN_E_HIP, "begin capture: %s", hipGetErrorString(e));
    }
    st = enqueue_decode(model, x, h, B, flags, layer_counts, nullptr, ws, cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    (void)hipStreamDestroy(cs);
    if (st) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (e != hipSuccess) return fail(SPFFN_E_HIP, "end capture: %s", hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return fail(SPFFN_E_HIP, "graph instantiate: %s", hipGetErrorString(e));
    }
    *out = new spffn_graph{graph, exec};
    return SPFFN_OK;
}

spffn_status spffn_graph_launch(const spffn_graph *graph, void *stream) {
    if (!graph) return fail(SPFFN_E_ARG, "graph_launch: NULL graph");
    SPFFN_HIP(hipGraphLaunch(graph->exec, (hipStream_t)stream), "graph launch");
    return SPFFN_OK;
}

void spffn_graph_destroy(spffn_graph *graph) {
    if (!graph) return;
    (void)hipGraphExecDestroy(graph->exec);
    (void)hipGraphDestroy(graph->graph);
    delete graph;
}

}  // extern "C"

namespace {

spffn_status check_decode_args(const spffn_model *model, const float *x, const float *h,
                               int32_t B, int32_t flags, const int32_t *layer_counts) {
    if (!model || !x || !h) return fail(SPFFN_E_ARG, "decode_step: NULL model, x or h");
    spffn_status st = check_batch(B);
    if (st) return st;
    if (flags & ~SPFFN_DECODE_DENSE) return fail(SPFFN_E_ARG, "decode_step: unknown flags");
    if (!aligned(x, 16) || !aligned(h, 16) || (layer_counts && !aligned(layer_counts, 4)))
        return fail(SPFFN_E_ARG, "decode_step: x and h must be 16-byte aligned");
    return SPFFN_OK;
}

spffn_status check_decode(const spffn_model *model, const float *x, const float *h, int32_t B,
                          int32_t flags, const int32_t *layer_counts, const void *ws,
                          size_t ws_bytes) {
    spffn_status st = check_decode_args(model, x, h, B, flags, layer_counts);
    if (st) return st;
    return check_ws(spffn_model_workspace_bytes(model, B), ws, ws_bytes);
}

spffn_status enqueue_decode(const spffn_model *model, const float *x, float *h, int32_t B,
                            int32_t flags, int32_t *layer_counts, const spffn_trace *trace,
                            void *ws, hipStream_t s, const float *tvec) {
    spffn_status st = SPFFN_OK;
    const bool dense = flags & SPFFN_DECODE_DENSE;
    const int d = model->d;
    {
        const Layer &L0 = model->layers[0]->L;
        if (B == 1 && !dense && model->uniform && single(L0, 1) && fused_fits(L0))
            return decode_one_token(model, x, h, layer_counts, trace, ws, tvec, s);
    }
    if (x != h) SPFFN_HIP(launch_copy_words(x, h, (int64_t)B * d, s), "input copy launch");
    size_t mask_off = 0, logit_off = 0;
    bool split_ready = false;  // w.xhi/xlo/ss already hold this layer's input split
    for (size_t l = 0; l < model->layers.size(); ++l) {
        const Layer &L = model->layers[l]->L;
        const int F = L.desc.d_ffn;
        Ws w = carve(L, B, ws);
        if (trace && trace->h_in)
            SPFFN_HIP(launch_copy_words(h, trace->h_in + l * (size_t)B * d, (int64_t)B * d, s),
                      "trace copy launch");
        const int32_t *idx = nullptr, *cnt = nullptr;
        float *lg = (trace && trace->logits) ? trace->logits + logit_off : nullptr;
        const bool one = single(L, B);
        // single token: the predictor's first kernel computes the RMS scale and
        // every kernel normalises on the fly; batches normalise into w.n first
        // (the matrix-core path also splits the normalised input into fp16 halves)
        const float *xin = one ? h : w.n;
        const bool mf = !one && mfma_fits(L, B);
        // Matrix-core layers of a sparse step chain: each layer's reduce also
        // writes the packed split of the raw h (and its sums of squares) that
        // the next one multiplies; the RMS scale is applied after the products.
        const bool chain = mf && !dense;
        bool next_chain = false;
        if (chain && l + 1 < model->layers.size()) {
            const Layer &Ln = model->layers[l + 1]->L;
            next_chain = !single(Ln, B) && mfma_fits(Ln, B);
        }
        if (chain) {
            if (!split_ready)
                SPFFN_HIP(launch_reduce_split(nullptr, 0, B, d, h, h, w.xhi, w.xlo, w.ss, s),
                          "split launch");
        } else if (mf) {
            SPFFN_HIP(launch_split_act(h, B, d, model->eps, true, w.n, w.xhi, w.xlo, s),
                      "rmsnorm launch");
        } else if (!one) {
            SPFFN_HIP(launch_rmsnorm(h, B, d, model->eps, w.n, s), "rmsnorm launch");
        }
        if (!dense) {
            // the matrix-core gather lists the union rows itself (from tile
            // masks of the predictor's last kernel); other paths compact
            if ((st = run_predict(L, xin, B, one, model->eps, lg, nullptr, w.uni, w, s, mf, mf,
                                  chain, tvec ? tvec + l * (size_t)B : nullptr)))
                return st;
            if (!mf)
                SPFFN_HIP(launch_compact(w.uni, F, w.idx, w.count, s,
                                         layer_counts ? layer_counts + l : nullptr),
                          "compact launch");
            if (trace && trace->union_mask)
                SPFFN_HIP(hipMemcpyAsync(trace->union_mask + mask_off, w.uni, F,
                                         hipMemcpyDeviceToDevice, s),
                          "trace copy");
            idx = w.idx;
            cnt = w.count;
        } else {
            if (one) SPFFN_HIP(launch_rms_scale(h, B, d, model->eps, w.scale, s), "rms launch");
            if (layer_counts)
                SPFFN_HIP(launch_fill_i32(layer_counts + l, F, 1, s), "count fill launch");
        }
        if (trace && trace->events)
            SPFFN_HIP(hipEventRecord((hipEvent_t)trace->events[2 * l], s), "event record");
        if ((st = run_ffn(L, xin, one ? w.scale : nullptr, B, idx, cnt, h, h, w, s, mf, chain,
                          layer_counts ? layer_counts + l : nullptr, chain, next_chain)))
            return st;
        split_ready = next_chain;
        if (trace && trace->events)
            SPFFN_HIP(hipEventRecord((hipEvent_t)trace->events[2 * l + 1], s), "event record");
        mask_off += F;
        logit_off += (size_t)B * F;
    }
    return SPFFN_OK;
}

}  // namespace

extern "C" {

spffn_status spffn_profile(const spffn_layer *layer, const float *x, int32_t N, int32_t *counts,
                           void *ws, size_t ws_bytes, void *stream) {
    if (!layer || !x || !counts) return fail(SPFFN_E_ARG, "profile: NULL pointer");
    if (N < 1) return fail(SPFFN_E_SHAPE, "profile: N=%d < 1", N);
    if (!aligned(x, 16) || !aligned(counts, 4)) return fail(SPFFN_E_ARG, "profile: misaligned");
    const Layer &L = layer->L;
    const size_t half_bytes = (size_t)16 * L.desc.d * sizeof(_Float16);
    if (ws && ws_bytes >= spffn_profile_workspace_bytes(layer) && aligned(ws, 256) &&
        mfma_profile_fits(L)) {
        _Float16 *hi = static_cast<_Float16 *>(ws);
        _Float16 *lo = reinterpret_cast<_Float16 *>(static_cast<char *>(ws) + half_bytes);
        SPFFN_HIP(launch_mfma_profile(L, x, N, counts, hi, lo, (hipStream_t)stream),
                  "profile launch");
        return SPFFN_OK;
    }
    const WMat &wa = L.desc.kind != SPFFN_RELU ? L.gate : L.up;
    SPFFN_HIP(launch_gemv_count(L.desc.w_dtype, wa, L.desc.d_ffn, L.desc.d, x, N, L.desc.b_act,
                                counts, (hipStream_t)stream),
              "profile launch");
    return SPFFN_OK;
}

size_t spffn_profile_workspace_bytes(const spffn_layer *layer) {
    return layer ? (size_t)2 * 16 * layer->L.desc.d * sizeof(_Float16) : 0;
}

spffn_status spffn_hot_first_order(const int32_t *counts, int32_t n, int32_t *perm,
                                   void *stream) {
    if (!counts || !perm) return fail(SPFFN_E_ARG, "hot_first_order: NULL pointer");
    if (n < 1) return fail(SPFFN_E_SHAPE, "hot_first_order: n=%d < 1", n);
    SPFFN_HIP(launch_hot_first_order(counts, n, perm, (hipStream_t)stream),
              "hot_first_order launch");
    return SPFFN_OK;
}

spffn_status spffn_permute_rows(const void *src, void *dst, const int32_t *perm, int32_t rows,
                                int64_t row_bytes, void *stream) {
    if (!src || !dst || !perm) return fail(SPFFN_E_ARG, "permute_rows: NULL pointer");
    if (rows < 1 || row_bytes < 4 || row_bytes % 4)
        return fail(SPFFN_E_SHAPE, "permute_rows: rows=%d row_bytes=%lld", rows,
                    (long long)row_bytes);
    if (!aligned(src, 4) || !aligned(dst, 4)) return fail(SPFFN_E_ARG, "permute_rows: misaligned");
    const uint8_t *s8 = static_cast<const uint8_t *>(src);
    uint8_t *d8 = static_cast<uint8_t *>(dst);
    const size_t bytes = (size_t)rows * (size_t)row_bytes;
    if (s8 < d8 + bytes && d8 < s8 + bytes)
        return fail(SPFFN_E_ARG, "permute_rows: src and dst overlap");
    SPFFN_HIP(launch_permute_rows(src, dst, perm, rows, row_bytes, (hipStream_t)stream),
              "permute_rows launch");
    return SPFFN_OK;
}

spffn_status spffn_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return fail(SPFFN_E_ARG, "stream_read: NULL pointer");
    if (bytes < 16 || bytes % 16)
        return fail(SPFFN_E_SHAPE, "stream_read: bytes=%lld must be a positive multiple of 16",
                    (long long)bytes);
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return fail(SPFFN_E_ARG, "stream_read: buf must be 16-byte, sink 4-byte aligned");
    SPFFN_HIP(launch_stream_read(buf, bytes, sink, (hipStream_t)stream), "stream_read launch");
    return SPFFN_OK;
}

spffn_status spffn_q4_0_repack(const void *aos, void *soa, int32_t rows, int32_t cols,
                               void *stream) {
    if (!aos || !soa) return fail(SPFFN_E_ARG, "q4_0_repack: NULL pointer");
    if (rows < 1 || cols < 32 || cols % 32)
        return fail(SPFFN_E_SHAPE, "q4_0_repack: rows=%d cols=%d (cols %% 32 == 0)", rows, cols);
    if (!aligned(aos, 2) || !aligned(soa, 16))
        return fail(SPFFN_E_ARG, "q4_0_repack: aos must be 2-byte, soa 16-byte aligned");
    SPFFN_HIP(launch_q4_0_repack(aos, soa, rows, cols, (hipStream_t)stream), "repack launch");
    return SPFFN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode step without a caller workspace.  Its kernels use this file-scope
// array instead: one copy per GPU, held until the process ends.  In host code
// the name `scratch` is only a stand-in for the symbol; the array's device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[SPFFN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices] = {};

// Device address of the current device's copy of `scratch`.
spffn_status scratch_address(void **out) {
    int dev = -1;
    SPFFN_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(SPFFN_E_ARG, "decode_step_noalloc: device %d outside [0, %d)", dev,
                    kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SPFFN_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return SPFFN_OK;
}

}  // namespace

extern "C" spffn_status spffn_decode_step_noalloc(const spffn_model *model, const float *x,
                                                  float *h, int32_t B, int32_t flags,
                                                  int32_t *layer_counts, void *stream) {
    spffn_status st = check_decode_args(model, x, h, B, flags, layer_counts);
    if (st) return st;
    const size_t need = spffn_model_workspace_bytes(model, B);
    if (need > (size_t)SPFFN_NOALLOC_SCRATCH_BYTES)
        return fail(SPFFN_E_WORKSPACE,
                    "decode_step_noalloc: this model needs %zu bytes of scratch at B=%d, more "
                    "than the library's static %zu-byte array (use spffn_decode_step with a "
                    "workspace)",
                    need, B, (size_t)SPFFN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_address(&ws))) return st;
    return enqueue_decode(model, x, h, B, flags, layer_counts, nullptr, ws, (hipStream_t)stream);
}
