// C ABI of libspffn: argument validation, workspace layout and the launch
// sequences of predict / forward / decode_step.  Every entry point validates
// before it enqueues anything and never synchronises the host.
#include <cmath>
#include <cstdarg>
#include <cstdio>
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

int elems_multiple(int dtype) { return dtype == SPFFN_F32 ? 4 : dtype == SPFFN_F16 ? 8 : 32; }

WMat wmat(const void *p, int dtype, int rows, int cols) {
    WMat w{};
    w.data = static_cast<const uint8_t *>(p);
    w.scales = nullptr;
    if (dtype == SPFFN_Q4_0 && p)
        w.scales = reinterpret_cast<const uint16_t *>(w.data + (size_t)rows * (cols / 2));
    return w;
}

struct Ws {
    float *n, *hid, *act, *part;
    uint8_t *mask, *uni;
    int32_t *idx, *count;
    int chunks;
};

Ws carve(const Layer &L, int B, void *ws) {
    WsLayout lo = layer_ws_layout(L, B);
    uint8_t *base = static_cast<uint8_t *>(ws);
    Ws w;
    w.n = reinterpret_cast<float *>(base + lo.n);
    w.hid = reinterpret_cast<float *>(base + lo.hid);
    w.mask = base + lo.mask;
    w.uni = base + lo.uni;
    w.idx = reinterpret_cast<int32_t *>(base + lo.idx);
    w.count = reinterpret_cast<int32_t *>(base + lo.count);
    w.act = reinterpret_cast<float *>(base + lo.act);
    w.part = reinterpret_cast<float *>(base + lo.part);
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

// The FFN part of one layer for B tokens over (idx, count) or every neuron.
spffn_status run_ffn(const Layer &L, const float *x, int B, const int32_t *idx,
                     const int32_t *count, const float *resid, float *y, const Ws &w,
                     hipStream_t s) {
    SPFFN_HIP(launch_ffn_up(L, x, B, idx, count, w.act, s), "gather up/gate launch");
    SPFFN_HIP(launch_ffn_down(L, B, idx, count, w.act, w.part, w.chunks, s),
              "gather down launch");
    SPFFN_HIP(launch_reduce(w.part, w.chunks, B, L.desc.d, resid, y, s), "reduce launch");
    return SPFFN_OK;
}

spffn_status run_predict(const Layer &L, const float *x, int B, float *logits, uint8_t *mask,
                         uint8_t *uni, const Ws &w, hipStream_t s) {
    const spffn_layer_desc &D = L.desc;
    SPFFN_HIP(launch_gemv_hid(D.p_dtype, L.w1, D.r, D.d, x, B, D.p_b1, w.hid, s),
              "predictor layer-1 launch");
    SPFFN_HIP(launch_gemv_mask(D.p_dtype, L.w2, D.d_ffn, D.r, w.hid, B, D.p_b2, L.t, logits, mask,
                               uni, s),
              "predictor layer-2 launch");
    return SPFFN_OK;
}

}  // namespace

namespace spffn {

WsLayout layer_ws_layout(const Layer &L, int B) {
    const spffn_layer_desc &D = L.desc;
    WsLayout lo{};
    lo.chunks = down_chunks(L);
    size_t off = 0;
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
    lo.act = off;
    off += up256((size_t)B * D.d_ffn * 4);
    lo.part = off;
    off += up256((size_t)lo.chunks * B * D.d * 4);
    lo.total = off;
    return lo;
}

}  // namespace spffn

extern "C" {

const char *spffn_last_error(void) { return g_err.c_str(); }

const char *spffn_version(void) { return "spffn 0.1 (gfx950)"; }

spffn_status spffn_layer_create(const spffn_layer_desc *desc, spffn_layer **out) {
    if (!desc || !out) return fail(SPFFN_E_ARG, "layer_create: NULL desc or out");
    const spffn_layer_desc &D = *desc;
    if (D.d <= 0 || D.d_ffn <= 0 || D.r <= 0)
        return fail(SPFFN_E_SHAPE, "layer_create: d=%d d_ffn=%d r=%d must be positive", D.d,
                    D.d_ffn, D.r);
    if (D.kind != SPFFN_RELU && D.kind != SPFFN_REGLU)
        return fail(SPFFN_E_ARG, "layer_create: unknown kind %d", D.kind);
    if (D.w_dtype != SPFFN_F32 && D.w_dtype != SPFFN_F16 && D.w_dtype != SPFFN_Q4_0)
        return fail(SPFFN_E_DTYPE, "layer_create: unknown weight dtype %d", D.w_dtype);
    if (D.p_dtype != SPFFN_F32 && D.p_dtype != SPFFN_F16)
        return fail(SPFFN_E_DTYPE, "layer_create: predictor dtype must be F32 or F16, got %d",
                    D.p_dtype);
    if (D.d % elems_multiple(D.w_dtype))
        return fail(SPFFN_E_SHAPE, "layer_create: d=%d must be a multiple of %d for dtype %d", D.d,
                    elems_multiple(D.w_dtype), D.w_dtype);
    if (D.d % elems_multiple(D.p_dtype) || D.r % elems_multiple(D.p_dtype))
        return fail(SPFFN_E_SHAPE, "layer_create: d=%d and r=%d must be multiples of %d", D.d, D.r,
                    elems_multiple(D.p_dtype));
    if (!(D.tau > 0.0f && D.tau < 1.0f))
        return fail(SPFFN_E_ARG, "layer_create: tau=%g outside (0, 1)", (double)D.tau);
    if (D.reserved != 0) return fail(SPFFN_E_ARG, "layer_create: reserved must be 0");
    if (!D.w_up || !D.w_down_t || !D.p_w1 || !D.p_b1 || !D.p_w2 || !D.p_b2)
        return fail(SPFFN_E_ARG, "layer_create: a required weight pointer is NULL");
    if (D.kind == SPFFN_REGLU && !D.w_gate)
        return fail(SPFFN_E_ARG, "layer_create: ReGLU needs w_gate");
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
    const double tau = (double)D.tau;
    h->L.t = (float)std::log(tau / (1.0 - tau));
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
    if (!aligned(x, 4) || (logits && !aligned(logits, 4)))
        return fail(SPFFN_E_ARG, "predict: misaligned x or logits");
    const Layer &L = layer->L;
    if ((st = check_ws(layer_ws_layout(L, B).total, ws, ws_bytes))) return st;
    Ws w = carve(L, B, ws);
    return run_predict(L, x, B, logits, mask, union_mask, w, (hipStream_t)stream);
}

spffn_status spffn_forward(const spffn_layer *layer, const float *x, int32_t B,
                           const uint8_t *mask, const int32_t *idx, const int32_t *count,
                           float *y, void *ws, size_t ws_bytes, void *stream) {
    if (!layer || !x || !y) return fail(SPFFN_E_ARG, "forward: NULL layer, x or y");
    spffn_status st = check_batch(B);
    if (st) return st;
    if (!aligned(x, 4) || !aligned(y, 4)) return fail(SPFFN_E_ARG, "forward: misaligned x or y");
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
    return run_ffn(L, x, B, use_idx, use_count, nullptr, y, w, s);
}

spffn_status spffn_decode_step(const spffn_model *model, const float *x, float *h, int32_t B,
                               int32_t flags, int32_t *layer_counts, const spffn_trace *trace,
                               void *ws, size_t ws_bytes, void *stream) {
    if (!model || !x || !h) return fail(SPFFN_E_ARG, "decode_step: NULL model, x or h");
    spffn_status st = check_batch(B);
    if (st) return st;
    if (flags & ~SPFFN_DECODE_DENSE) return fail(SPFFN_E_ARG, "decode_step: unknown flags");
    if (!aligned(x, 4) || !aligned(h, 4) || (layer_counts && !aligned(layer_counts, 4)))
        return fail(SPFFN_E_ARG, "decode_step: misaligned pointer");
    if ((st = check_ws(spffn_model_workspace_bytes(model, B), ws, ws_bytes))) return st;
    const bool dense = flags & SPFFN_DECODE_DENSE;
    hipStream_t s = (hipStream_t)stream;
    const int d = model->d;
    if (x != h) SPFFN_HIP(launch_copy_words(x, h, (int64_t)B * d, s), "input copy launch");
    size_t mask_off = 0, logit_off = 0;
    for (size_t l = 0; l < model->layers.size(); ++l) {
        const Layer &L = model->layers[l]->L;
        const int F = L.desc.d_ffn;
        Ws w = carve(L, B, ws);
        if (trace && trace->h_in)
            SPFFN_HIP(launch_copy_words(h, trace->h_in + l * (size_t)B * d, (int64_t)B * d, s),
                      "trace copy launch");
        SPFFN_HIP(launch_rmsnorm(h, B, d, model->eps, w.n, s), "rmsnorm launch");
        const int32_t *idx = nullptr, *cnt = nullptr;
        if (!dense) {
            float *lg = (trace && trace->logits) ? trace->logits + logit_off : nullptr;
            if ((st = run_predict(L, w.n, B, lg, nullptr, w.uni, w, s))) return st;
            SPFFN_HIP(launch_compact(w.uni, F, w.idx, w.count, s), "compact launch");
            if (trace && trace->union_mask)
                SPFFN_HIP(hipMemcpyAsync(trace->union_mask + mask_off, w.uni, F,
                                         hipMemcpyDeviceToDevice, s),
                          "trace copy");
            idx = w.idx;
            cnt = w.count;
            if (layer_counts)
                SPFFN_HIP(launch_copy_words(w.count, layer_counts + l, 1, s), "count copy launch");
        } else if (layer_counts) {
            SPFFN_HIP(launch_fill_i32(layer_counts + l, F, 1, s), "count fill launch");
        }
        if ((st = run_ffn(L, w.n, B, idx, cnt, h, h, w, s))) return st;
        mask_off += F;
        logit_off += (size_t)B * F;
    }
    return SPFFN_OK;
}

spffn_status spffn_profile(const spffn_layer *layer, const float *x, int32_t N, int32_t *counts,
                           void *ws, size_t ws_bytes, void *stream) {
    (void)ws;
    (void)ws_bytes;
    if (!layer || !x || !counts) return fail(SPFFN_E_ARG, "profile: NULL pointer");
    if (N < 1) return fail(SPFFN_E_SHAPE, "profile: N=%d < 1", N);
    if (!aligned(x, 4) || !aligned(counts, 4)) return fail(SPFFN_E_ARG, "profile: misaligned");
    const Layer &L = layer->L;
    const WMat &wa = L.desc.kind == SPFFN_REGLU ? L.gate : L.up;
    SPFFN_HIP(launch_gemv_count(L.desc.w_dtype, wa, L.desc.d_ffn, L.desc.d, x, N, L.desc.b_act,
                                counts, (hipStream_t)stream),
              "profile launch");
    return SPFFN_OK;
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
