// Device helpers for the row-streaming kernels of libspffn (gfx950, wave64).
//
// Every weight row is read as 16-byte "packets", one per lane per step, so a
// wave moves 1 KiB of weights per load instruction (128-bit loads, fully
// coalesced).  A packet is 4 fp32, 8 fp16, or one 4-bit block of 32 codes.
//
// Activations are staged in LDS in a packet-transposed layout so that lane p
// reads the values for its packet as float4s at consecutive addresses (no bank
// conflicts):  for a chunk of NP packets of E elements,
//     xl[b * NP*E + (g * NP + p) * 4 + n] = x[b][c0 + p*E + 4*g + n]
// with g < E/4, n < 4.  For 4-bit packets the per-block sums of x are kept too
// (xsum[b * NP + p]), so a block's dot product is  s * (sum q_k x_k - 8 sum x_k).
#pragma once

#include <type_traits>

#include "internal.h"

namespace spffn {

template <int FMT> struct PacketElems;
template <> struct PacketElems<kF32> { static constexpr int value = 4; };
template <> struct PacketElems<kF16> { static constexpr int value = 8; };
template <> struct PacketElems<kQ4> { static constexpr int value = 32; };
template <> struct PacketElems<kFP8> { static constexpr int value = 16; };

inline int packet_elems(int fmt) {
    return fmt == kF32 ? 4 : fmt == kF16 ? 8 : fmt == kFP8 ? 16 : 32;
}

// Bytes of one stored row of `cols` elements.
template <int FMT>
__host__ __device__ __forceinline__ size_t row_bytes(int cols) {
    return FMT == kF32 ? (size_t)cols * 4
           : FMT == kF16 ? (size_t)cols * 2
           : FMT == kFP8 ? (size_t)cols
                         : (size_t)cols / 2;
}

template <int FMT>
__device__ __forceinline__ const uint4 *row_ptr(const WMat &w, size_t row, int cols) {
    (void)cols;
    return reinterpret_cast<const uint4 *>(w.data + row * w.stride);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// fp8 (OCP E4M3) codes are widened as value / 256: the code's sign and its
// seven magnitude bits are moved under the binary16 sign, exponent and
// mantissa (E4M3 has exponent bias 7, binary16 bias 15, so every E4M3 value,
// subnormals included, is exactly 2^8 times the binary16 value so formed;
// the NaN codes 0x7F / 0xFF are not supported and read as +-480).  The 2^8
// goes into the row scale, so the scale a kernel applies is rscale * 256.
template <int FMT>
__device__ __forceinline__ float row_scale(const WMat &w, size_t row) {
    if constexpr (FMT == kFP8)
        return w.rscale[row] * 256.0f;
    else
        return 1.0f;
}

template <int FMT>
__device__ __forceinline__ float packet_scale(const WMat &w, size_t row, int cols, int pg) {
    if constexpr (FMT == kQ4)
        return half_bits_to_float(w.scales[row * (size_t)(cols / 32) + pg]);
    else if constexpr (FMT == kFP8)
        return row_scale<kFP8>(w, row);
    else
        return 1.0f;
}

// The four E4M3 codes of a 32-bit word (byte n = code n) as value / 256.
__device__ __forceinline__ void e4m3x4_div256(uint32_t w, float (&v)[4]) {
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const uint32_t x01 = __builtin_amdgcn_perm(0u, w, 0x0c010c00u);  // code 0 | code 1 << 16
    const uint32_t x23 = __builtin_amdgcn_perm(0u, w, 0x0c030c02u);  // code 2 | code 3 << 16
    const uint32_t h01 = ((x01 & 0x007F007Fu) << 7) | ((x01 & 0x00800080u) << 8);
    const uint32_t h23 = ((x23 & 0x007F007Fu) << 7) | ((x23 & 0x00800080u) << 8);
    const half2v a = __builtin_bit_cast(half2v, h01), b = __builtin_bit_cast(half2v, h23);
    v[0] = (float)a[0];
    v[1] = (float)a[1];
    v[2] = (float)b[0];
    v[3] = (float)b[1];
}

// Byte n (0..3) of a 32-bit word as a float, written so that it compiles to
// one v_cvt_f32_ubyte<n> (4-bit codes are widened a byte at a time).
__device__ __forceinline__ float byte_to_float(uint32_t w, int n) {
    typedef unsigned char uchar4v __attribute__((ext_vector_type(4)));
    const uchar4v b = __builtin_bit_cast(uchar4v, w);
    return (float)b[n];
}

// w & mask as one v_and_b32 the compiler cannot split into per-byte bit-field
// extracts, so that each byte is then widened by a single v_cvt_f32_ubyte<n>.
__device__ __forceinline__ uint32_t and_word(uint32_t w, uint32_t mask) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(mask), "v"(w));
    return r;
}

// Activation of the activated projection z: ReLU, or for SwiGLU layers the
// SiLU z * sigmoid(z) = z / (1 + e^-z) (z -> -inf gives -0, z -> +inf gives z).
__device__ __forceinline__ float gate_act(float z, bool silu) {
    return silu ? z / (1.0f + __expf(-z)) : fmaxf(z, 0.0f);
}

// Sum over the 64 lanes, returned to every lane: within each row of 16 lanes
// by DPP exchanges (pairs, quads, half-row and row mirrors; register-to-register,
// no LDS round trip), then the four row sums in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                          0xF, 0xF, false));
    };
    v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
    const int iv = __float_as_int(v);
    return (__int_as_float(__builtin_amdgcn_readlane(iv, 0)) +
            __int_as_float(__builtin_amdgcn_readlane(iv, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(iv, 32)) +
            __int_as_float(__builtin_amdgcn_readlane(iv, 48)));
}

// Stage tokens x[b][c0 .. c0 + NP*E) for b < NB (zeros for b >= B) into LDS.
// Call between barriers; when `xsum` is given, a second barrier-separated
// pass (stage_xsum) fills the 4-bit block sums.
template <int E, int NB>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int B, int ld, int c0, int NP,
                                        float *xl) {
    const int ncols = NP * E;
    for (int t = threadIdx.x; t < NB * ncols; t += blockDim.x) {
        const int b = t / ncols, c = t - b * ncols;
        const float v = (b < B) ? x[(size_t)b * ld + c0 + c] : 0.0f;
        const int p = c / E, k = c - p * E;
        xl[b * ncols + ((k >> 2) * NP + p) * 4 + (k & 3)] = v;
    }
}

template <int E, int NB>
__device__ __forceinline__ void stage_xsum(const float *xl, int NP, float *xsum) {
    const int ncols = NP * E;
    for (int t = threadIdx.x; t < NB * NP; t += blockDim.x) {
        const int b = t / NP, p = t - b * NP;
        const float *base = xl + b * ncols;
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < E / 4; ++g) {
            const float4 v = *reinterpret_cast<const float4 *>(base + (g * NP + p) * 4);
            s += v.x;
            s += v.y;
            s += v.z;
            s += v.w;
        }
        xsum[t] = s;
    }
}

__device__ __forceinline__ float4 lds4(const float *xl, int NP, int g, int p) {
    return *reinterpret_cast<const float4 *>(xl + (g * NP + p) * 4);
}

// acc[b] += dot(packet, x_b restricted to the packet's columns).
template <int FMT, int NB>
__device__ __forceinline__ void packet_dot(const uint4 raw, float scale, const float *xl, int NP,
                                           int p, const float *xsum, float (&acc)[NB]) {
    constexpr int E = PacketElems<FMT>::value;
    const int XS = NP * E;
    if constexpr (FMT == kF32) {
        const float w0 = __uint_as_float(raw.x), w1 = __uint_as_float(raw.y);
        const float w2 = __uint_as_float(raw.z), w3 = __uint_as_float(raw.w);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float4 v = lds4(xl + b * XS, NP, 0, p);
            float a = acc[b];
            a = fmaf(w0, v.x, a);
            a = fmaf(w1, v.y, a);
            a = fmaf(w2, v.z, a);
            a = fmaf(w3, v.w, a);
            acc[b] = a;
        }
    } else if constexpr (FMT == kF16) {
        typedef _Float16 half8 __attribute__((ext_vector_type(8)));
        const half8 h = __builtin_bit_cast(half8, raw);
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (float)h[e];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float4 v0 = lds4(xl + b * XS, NP, 0, p);
            const float4 v1 = lds4(xl + b * XS, NP, 1, p);
            float a = acc[b];
            a = fmaf(w[0], v0.x, a);
            a = fmaf(w[1], v0.y, a);
            a = fmaf(w[2], v0.z, a);
            a = fmaf(w[3], v0.w, a);
            a = fmaf(w[4], v1.x, a);
            a = fmaf(w[5], v1.y, a);
            a = fmaf(w[6], v1.z, a);
            a = fmaf(w[7], v1.w, a);
            acc[b] = a;
        }
    } else if constexpr (FMT == kFP8) {
        // 16 codes, word m holding columns 4m..4m+3; scale = rscale * 256
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        float w[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float v4[4];
            e4m3x4_div256(words[m], v4);
#pragma unroll
            for (int n = 0; n < 4; ++n) w[4 * m + n] = v4[n];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float a = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = lds4(xl + b * XS, NP, g, p);
                a = fmaf(w[4 * g + 0], v.x, a);
                a = fmaf(w[4 * g + 1], v.y, a);
                a = fmaf(w[4 * g + 2], v.z, a);
                a = fmaf(w[4 * g + 3], v.w, a);
            }
            acc[b] = fmaf(scale, a, acc[b]);
        }
    } else {
        // 4-bit block: word m holds codes 4m..4m+3 in its low nibbles (group m)
        // and codes 16+4m..16+4m+3 in its high nibbles (group 4+m).
        // low nibbles as bytes (q), high nibbles kept in place (16 q): both are
        // exact in fp32, and the high sum is scaled by 1/16 exactly at the end
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        float q[32];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = and_word(words[m], 0x0F0F0F0Fu);
            const uint32_t hi = and_word(words[m], 0xF0F0F0F0u);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                q[4 * m + n] = byte_to_float(lo, n);
                q[16 + 4 * m + n] = byte_to_float(hi, n);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float sl = 0.0f, sh = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = lds4(xl + b * XS, NP, g, p);
                sl = fmaf(q[4 * g + 0], v.x, sl);
                sl = fmaf(q[4 * g + 1], v.y, sl);
                sl = fmaf(q[4 * g + 2], v.z, sl);
                sl = fmaf(q[4 * g + 3], v.w, sl);
            }
#pragma unroll
            for (int g = 4; g < 8; ++g) {
                const float4 v = lds4(xl + b * XS, NP, g, p);
                sh = fmaf(q[4 * g + 0], v.x, sh);
                sh = fmaf(q[4 * g + 1], v.y, sh);
                sh = fmaf(q[4 * g + 2], v.z, sh);
                sh = fmaf(q[4 * g + 3], v.w, sh);
            }
            const float sq = fmaf(sh, 0.0625f, sl);
            acc[b] = fmaf(scale, fmaf(-8.0f, xsum[b * NP + p], sq), acc[b]);
        }
    }
}

// Register-operand forms: the E activation values of a packet are held by the
// lane itself (x[e] = column e of the packet), with their sum for 4-bit blocks.
template <int FMT>
__device__ __forceinline__ void load_packet_x(const float *__restrict__ x, int p,
                                              float (&xv)[PacketElems<FMT>::value], float &xsum) {
    constexpr int E = PacketElems<FMT>::value;
    const float4 *src = reinterpret_cast<const float4 *>(x + (size_t)p * E);
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
        const float4 v = src[g];
        xv[4 * g + 0] = v.x;
        xv[4 * g + 1] = v.y;
        xv[4 * g + 2] = v.z;
        xv[4 * g + 3] = v.w;
    }
    xsum = 0.0f;
    if constexpr (FMT == kQ4) {
#pragma unroll
        for (int e = 0; e < E; ++e) xsum += xv[e];
    }
}

// acc += dot(packet, x) with x in registers.
template <int FMT>
__device__ __forceinline__ float packet_dot_reg(const uint4 raw, float scale,
                                                const float (&xv)[PacketElems<FMT>::value],
                                                float xsum, float acc) {
    if constexpr (FMT == kF32) {
        acc = fmaf(__uint_as_float(raw.x), xv[0], acc);
        acc = fmaf(__uint_as_float(raw.y), xv[1], acc);
        acc = fmaf(__uint_as_float(raw.z), xv[2], acc);
        acc = fmaf(__uint_as_float(raw.w), xv[3], acc);
        return acc;
    } else if constexpr (FMT == kF16) {
        typedef _Float16 half8 __attribute__((ext_vector_type(8)));
        const half8 h = __builtin_bit_cast(half8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)h[e], xv[e], acc);
        return acc;
    } else if constexpr (FMT == kFP8) {
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        float s = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float v4[4];
            e4m3x4_div256(words[m], v4);
#pragma unroll
            for (int n = 0; n < 4; ++n) s = fmaf(v4[n], xv[4 * m + n], s);
        }
        return fmaf(scale, s, acc);
    } else {
        // low nibbles as bytes (q), high nibbles in place (16 q), see packet_dot
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        float sl = 0.0f, sh = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = and_word(words[m], 0x0F0F0F0Fu);
#pragma unroll
            for (int n = 0; n < 4; ++n) sl = fmaf(byte_to_float(lo, n), xv[4 * m + n], sl);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t hi = and_word(words[m], 0xF0F0F0F0u);
#pragma unroll
            for (int n = 0; n < 4; ++n) sh = fmaf(byte_to_float(hi, n), xv[16 + 4 * m + n], sh);
        }
        return fmaf(scale, fmaf(-8.0f, xsum, fmaf(sh, 0.0625f, sl)), acc);
    }
}

// Unpack one packet into E fp32 weights (used by the down projection, which
// scales whole rows rather than dotting them).
template <int FMT>
__device__ __forceinline__ void packet_values(const uint4 raw, float scale,
                                              float (&w)[PacketElems<FMT>::value]) {
    if constexpr (FMT == kF32) {
        w[0] = __uint_as_float(raw.x);
        w[1] = __uint_as_float(raw.y);
        w[2] = __uint_as_float(raw.z);
        w[3] = __uint_as_float(raw.w);
    } else if constexpr (FMT == kF16) {
        typedef _Float16 half8 __attribute__((ext_vector_type(8)));
        const half8 h = __builtin_bit_cast(half8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (float)h[e];
    } else {
        // (q - 8) s, with the high nibbles read in place as 16 q: 16 q s / 16
        // - 8 s is computed as (16 q - 128) (s / 16), exact up to the one rounding
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        const float s16 = scale * 0.0625f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = and_word(words[m], 0x0F0F0F0Fu);
            const uint32_t hi = and_word(words[m], 0xF0F0F0F0u);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                w[4 * m + n] = (byte_to_float(lo, n) - 8.0f) * scale;
                w[16 + 4 * m + n] = (byte_to_float(hi, n) - 128.0f) * s16;
            }
        }
    }
}

// acc[e] += a * (weight e of the packet).  For 4-bit packets the "- 8" of every
// code is left out and summed in `corr` instead (corr += a * scale), so each
// weight costs one widening and one multiply-add; the caller finishes with
// acc[e] -= 8 corr.  High nibbles are read in place (16 q) against a / 16,
// which gives the same product as q against a.
template <int FMT>
__device__ __forceinline__ void packet_axpy(const uint4 raw, float scale, float a,
                                            float (&acc)[PacketElems<FMT>::value], float &corr) {
    if constexpr (FMT == kQ4) {
        const float as = a * scale, as16 = as * 0.0625f;
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = and_word(words[m], 0x0F0F0F0Fu);
            const uint32_t hi = and_word(words[m], 0xF0F0F0F0u);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                acc[4 * m + n] = fmaf(as, byte_to_float(lo, n), acc[4 * m + n]);
                acc[16 + 4 * m + n] = fmaf(as16, byte_to_float(hi, n), acc[16 + 4 * m + n]);
            }
        }
        corr += as;
    } else {
        float w[PacketElems<FMT>::value];
        packet_values<FMT>(raw, scale, w);
#pragma unroll
        for (int e = 0; e < PacketElems<FMT>::value; ++e) acc[e] = fmaf(a, w[e], acc[e]);
    }
}

// Finish packet_axpy's accumulation: apply the summed "- 8" of 4-bit codes.
template <int FMT>
__device__ __forceinline__ void packet_axpy_finish(float (&acc)[PacketElems<FMT>::value],
                                                   float corr) {
    if constexpr (FMT == kQ4) {
#pragma unroll
        for (int e = 0; e < PacketElems<FMT>::value; ++e) acc[e] = fmaf(-8.0f, corr, acc[e]);
    }
}

// Column of packet element e within its row: packets hold consecutive columns,
// except 4-bit blocks, whose element order is already the column order
// (code k is column k of the block).
template <int FMT>
__device__ __forceinline__ int packet_col(int p, int e) {
    return p * PacketElems<FMT>::value + e;
}

}  // namespace spffn
