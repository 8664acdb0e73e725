// conv.hip -- ssd_conv_fwd: causal depthwise conv (k = 4) + activation over
// the [x | B | C] columns, and dt = softplus(dt_raw + dt_bias), on gfx950.
//
// Layout of the work: two 64-lane waves per block; lane l owns 16 bytes of
// channels (8 bf16 or 4 fp32) and walks a tile of kTile consecutive tokens
// with the last three raw rows in registers, so every raw row is read once
// (plus a 3-row halo per tile) and every output row written once, in 2 KiB
// coalesced row segments per block (measured 3-6 % faster than one wave per
// block; whole rows per block, 6 waves at conv_dim 3072, measured 30 % slower).  A ring of kBatch rows is kept loading ahead of
// the row being convolved.  SiLU uses the hardware exp2 and reciprocal (a
// few fp32 ulp, far inside one bf16 ulp).  An extra column of blocks
// (blockIdx.x == number of channel blocks) computes dt for the same tokens,
// in 16-byte pieces when the heads and rows line up (else element by
// element), with several loads per lane in flight.
//
// Document isolation (Mini-K3-1H card, "Checkpoint and training": the conv
// history resets at every document boundary): when token t starts a new
// document, the three history registers are zeroed before t is convolved,
// so no value from an earlier document reaches t or any later token by any
// arithmetic path.  The carried conv state only ever sits in the history
// registers of tile 0, so it reaches exactly the tokens before the row's
// first boundary.
//
// Tap order: conv_w[c][3] multiplies the current token (the un-reversed form
// of the [conv_dim, 1, d_conv] weight listed by the Codestral-Mamba port).
#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kConvThreads = 128;   // two waves: 2 KiB of each bf16 row per block
constexpr int kTile = 64;     // tokens per block (a multiple of 64)
constexpr int kStartWords = kTile / 64;
constexpr int kBatch = 16;    // rows loaded before use
// the ring below refills slot u with the row kBatch further on: whole tiles
// must be a whole number of rings, or the last refills run past the tile
static_assert(kTile % kBatch == 0 && kTile >= kBatch, "a tile is a whole number of load rings");
constexpr int kDtBatch = 8;   // dt elements loaded per lane before use

template <typename T> struct CV;
template <> struct CV<float> {
    static constexpr int n = 4;
    __device__ static void unpack(uint4 v, float* o) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
    __device__ static uint4 pack(const float* o) {
        return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
    }
    __device__ static float scalar(const void* p, size_t i) { return static_cast<const float*>(p)[i]; }
};
template <> struct CV<uint16_t> {
    static constexpr int n = 8;
    __device__ static void unpack(uint4 v, float* o) {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
    }
    __device__ static uint4 pack(const float* o) {
        return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                          pack_bf16x2(o[6], o[7]));
    }
    __device__ static float scalar(const void* p, size_t i) { return bf16_to_f32(static_cast<const uint16_t*>(p)[i]); }
};

__device__ __forceinline__ bool is_boundary(const int32_t* doc, int t) {
    return doc != nullptr && t > 0 && doc[t] != doc[t - 1];
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void ssd_conv_kernel(ConvArgs a) {
    constexpr int VEC = CV<T>::n;
    const int C = a.C, L = a.L;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * kTile;
    const int t1 = min(t0 + kTile, L);
    const int ncb = (C / VEC + kConvThreads - 1) / kConvThreads;
    const int32_t* doc = a.doc ? a.doc + (size_t)b * a.Lb_in : nullptr;

    if ((int)blockIdx.x == ncb) {
        // ---- dt = softplus(dt_raw + dt_bias) for the tile's tokens
        if (a.dt_raw == nullptr) return;
        const int H = a.H;
        // 16-byte pieces: a lane takes DV consecutive heads of one token when
        // the heads, the row stride and the three arrays line up
        constexpr int DV = 16 / sizeof(T);
        const bool vec = H % DV == 0 && a.dt_stride % DV == 0 && (reinterpret_cast<uintptr_t>(a.dt_raw) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(a.dt_out) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(a.dt_bias) & 15) == 0;
        if (vec) {
            const int hv = H / DV;               // pieces per token
            const int n = (t1 - t0) * hv;
            for (int i0 = threadIdx.x; i0 < n; i0 += kDtBatch * kConvThreads) {
                uint4 r[kDtBatch];
#pragma unroll
                for (int u = 0; u < kDtBatch; ++u) {
                    const int i = min(i0 + u * kConvThreads, n - 1);
                    r[u] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.dt_raw) +
                                                           ((size_t)b * a.Lb_in + t0 + i / hv) * a.dt_stride +
                                                           (i % hv) * DV);
                }
#pragma unroll
                for (int u = 0; u < kDtBatch; ++u) {
                    const int i = i0 + u * kConvThreads;
                    if (i < n) {
                        const int h = (i % hv) * DV;
                        float v[DV];
                        CV<T>::unpack(r[u], v);
                        float* o = a.dt_out + ((size_t)b * a.Lb_out + t0 + i / hv) * H + h;
#pragma unroll
                        for (int e = 0; e < DV; e += 4) {
                            float4 bb = make_float4(0.f, 0.f, 0.f, 0.f);
                            if (a.dt_bias) bb = *reinterpret_cast<const float4*>(a.dt_bias + h + e);
                            *reinterpret_cast<float4*>(o + e) =
                                make_float4(softplus_f(v[e] + bb.x), softplus_f(v[e + 1] + bb.y),
                                            softplus_f(v[e + 2] + bb.z), softplus_f(v[e + 3] + bb.w));
                        }
                    }
                }
            }
            return;
        }
        const int n = (t1 - t0) * H;
        // kDtBatch independent loads per lane are in flight before any is used
        // (indices clamp to the last element, whose store alone is kept)
        for (int i0 = threadIdx.x; i0 < n; i0 += kDtBatch * kConvThreads) {
            float r[kDtBatch];
#pragma unroll
            for (int u = 0; u < kDtBatch; ++u) {
                const int i = min(i0 + u * kConvThreads, n - 1);
                r[u] = CV<T>::scalar(a.dt_raw, ((size_t)b * a.Lb_in + t0 + i / H) * a.dt_stride + i % H);
            }
#pragma unroll
            for (int u = 0; u < kDtBatch; ++u) {
                const int i = i0 + u * kConvThreads;
                if (i < n) {
                    const int h = i % H;
                    a.dt_out[((size_t)b * a.Lb_out + t0 + i / H) * H + h] =
                        softplus_f(r[u] + (a.dt_bias ? a.dt_bias[h] : 0.0f));
                }
            }
        }
        return;
    }

    // document starts inside the tile as a bit mask (bit i of word j: token
    // t0 + 64 j + i starts a document), one doc-id pair per lane and word;
    // built before any lane leaves
    uint64_t starts[kStartWords] = {};
    if (doc) {
#pragma unroll
        for (int j = 0; j < kStartWords; ++j) {
            const int tj = t0 + 64 * j + (int)(threadIdx.x % 64);   // every wave builds the same mask
            const int tt = min(tj, t1 - 1);
            const bool s_here = tj < t1 && tt > 0 && doc[tt] != doc[tt - 1];
            starts[j] = __ballot(s_here);
        }
    }

    const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * VEC;
    if (c0 >= C) return;
    const T* raw = static_cast<const T*>(a.raw) + (size_t)b * a.Lb_in * a.raw_stride + c0;
    T* out = static_cast<T*>(a.out) + (size_t)b * a.Lb_out * a.out_stride + c0;

    float w[4][VEC], bias[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float4 wv = *reinterpret_cast<const float4*>(a.w + (size_t)(c0 + e) * 4);
        w[0][e] = wv.x; w[1][e] = wv.y; w[2][e] = wv.z; w[3][e] = wv.w;
        bias[e] = a.bias ? a.bias[c0 + e] : 0.0f;
    }

    // history registers: h3 = tap t-3, h2 = t-2, h1 = t-1
    float h3[VEC], h2[VEC], h1[VEC];
    if (t0 == 0) {
        const T* st = a.state_in ? static_cast<const T*>(a.state_in) + (size_t)b * 3 * C + c0 : nullptr;
        if (st) {
            CV<T>::unpack(*reinterpret_cast<const uint4*>(st), h3);
            CV<T>::unpack(*reinterpret_cast<const uint4*>(st + C), h2);
            CV<T>::unpack(*reinterpret_cast<const uint4*>(st + 2 * C), h1);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) h3[e] = h2[e] = h1[e] = 0.0f;
        }
    } else {
        // t0 >= kTile >= 3: the halo rows exist; boundaries inside the halo cut older taps
        CV<T>::unpack(*reinterpret_cast<const uint4*>(raw + (size_t)(t0 - 3) * a.raw_stride), h3);
        CV<T>::unpack(*reinterpret_cast<const uint4*>(raw + (size_t)(t0 - 2) * a.raw_stride), h2);
        CV<T>::unpack(*reinterpret_cast<const uint4*>(raw + (size_t)(t0 - 1) * a.raw_stride), h1);
        if (is_boundary(doc, t0 - 2)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) h3[e] = 0.0f;
        }
        if (is_boundary(doc, t0 - 1)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) h3[e] = h2[e] = 0.0f;
        }
    }

    // raw rows are read once (the halo aside): nontemporal loads keep them from
    // displacing the conv output the scan reads next.
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    auto load_row = [&](int t) {
        const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(raw + (size_t)t * a.raw_stride));
        return make_uint4(q.x, q.y, q.z, q.w);
    };
    auto conv_row = [&](const uint4& rv, int t) {
        float cur[VEC], o[VEC];
        CV<T>::unpack(rv, cur);
        if ((starts[(t - t0) >> 6] >> ((t - t0) & 63)) & 1) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) h3[e] = h2[e] = h1[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float v = bias[e];
            v = fmaf(w[0][e], h3[e], v);
            v = fmaf(w[1][e], h2[e], v);
            v = fmaf(w[2][e], h1[e], v);
            v = fmaf(w[3][e], cur[e], v);
            if (a.act == 0) v = silu_f(v);
            o[e] = v;
            h3[e] = h2[e];
            h2[e] = h1[e];
            h1[e] = cur[e];
        }
        *reinterpret_cast<uint4*>(out + (size_t)t * a.out_stride) = CV<T>::pack(o);
    };
    if (t1 - t0 == kTile) {
        // a ring of kBatch row slots kept full: slot u, once consumed, is
        // refilled with the row kBatch further on (every load and store is
        // unconditional, so kBatch loads stay in flight through the tile)
        uint4 rows[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) rows[u] = load_row(t0 + u);
        for (int tb = t0; tb < t1 - kBatch; tb += kBatch) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const uint4 rv = rows[u];
                rows[u] = load_row(tb + kBatch + u);
                conv_row(rv, tb + u);
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) conv_row(rows[u], t1 - kBatch + u);
    } else {
        for (int t = t0; t < t1; ++t) conv_row(load_row(t), t);
    }

    // ---- conv state after the call (tile 0 owns it: it alone read state_in)
    if (t0 == 0 && a.state_out != nullptr) {
        float s0[VEC], s1[VEC], s2[VEC];
        if (t1 == L) {
            // this lane convolved the last token: its history registers are the state
#pragma unroll
            for (int e = 0; e < VEC; ++e) { s0[e] = h3[e]; s1[e] = h2[e]; s2[e] = h1[e]; }
        } else {
            // L > kTile >= 3: the last three raw rows, cut at boundaries inside them
            CV<T>::unpack(*reinterpret_cast<const uint4*>(raw + (size_t)(L - 3) * a.raw_stride), s0);
            CV<T>::unpack(*reinterpret_cast<const uint4*>(raw + (size_t)(L - 2) * a.raw_stride), s1);
            CV<T>::unpack(*reinterpret_cast<const uint4*>(raw + (size_t)(L - 1) * a.raw_stride), s2);
            if (is_boundary(doc, L - 2)) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) s0[e] = 0.0f;
            }
            if (is_boundary(doc, L - 1)) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) s0[e] = s1[e] = 0.0f;
            }
        }
        T* so = static_cast<T*>(a.state_out) + (size_t)b * 3 * C + c0;
        *reinterpret_cast<uint4*>(so) = CV<T>::pack(s0);
        *reinterpret_cast<uint4*>(so + C) = CV<T>::pack(s1);
        *reinterpret_cast<uint4*>(so + 2 * C) = CV<T>::pack(s2);
    }
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.L == 0) {
        // nothing to convolve; a requested state_out is the (possibly absent) state_in
        return hipSuccess;
    }
    const int vec = a.dtype == 0 ? 4 : 8;
    const int ncb = (a.C / vec + kConvThreads - 1) / kConvThreads;
    dim3 grid(ncb + 1, (a.L + kTile - 1) / kTile, a.B);
    if (a.dtype == 0)
        hipLaunchKernelGGL(ssd_conv_kernel<float>, grid, dim3(kConvThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(ssd_conv_kernel<uint16_t>, grid, dim3(kConvThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ssd

namespace ssd {

namespace {
__global__ void copy16_kernel(const uint4* src, uint4* dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : make_uint4(0, 0, 0, 0);
}
}  // namespace

__global__ void copy_rows_kernel(const char* src, int64_t srs, int64_t sbs, char* dst, int64_t drs, int64_t dbs,
                                 int rows, int row_words) {
    const int b = blockIdx.y;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (int64_t)rows * row_words;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(i / row_words), w = (int)(i % row_words);
        *reinterpret_cast<uint4*>(dst + b * dbs + r * drs + 16 * w) =
            *reinterpret_cast<const uint4*>(src + b * sbs + r * srs + 16 * w);
    }
}

// Rows t >= lengths[b] of y (fp32 [B][L][width], rows `stride` floats apart)
// set to +0.0; one workgroup per (64-row tile, batch row).  lengths are read
// on the device and clamped to [0, L].
__global__ void zero_rows_kernel(float* y, int64_t stride, int L, int width4, const int32_t* lengths) {
    const int b = blockIdx.y, t0 = blockIdx.x * 64;
    const int len = min(max(lengths[b], 0), L);
    const int r0 = max(t0, len), r1 = min(t0 + 64, L);
    for (int64_t i = threadIdx.x; i < (int64_t)(r1 - r0) * width4; i += blockDim.x) {
        const int r = r0 + (int)(i / width4), w = (int)(i % width4);
        *reinterpret_cast<float4*>(y + ((int64_t)b * L + r) * stride + 4 * w) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

hipError_t launch_zero_rows(float* y, int64_t stride, int B, int L, int width, const int32_t* lengths,
                            hipStream_t stream) {
    if (B == 0 || L == 0 || width == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((L + 63) / 64, B), dim3(256), 0, stream, y, stride, L, width / 4,
                       lengths);
    return hipGetLastError();
}

hipError_t launch_copy16(const void* src, void* dst, size_t n, hipStream_t stream) {
    if (n == 0 || src == dst) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(copy16_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), n);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int64_t src_row_stride, int64_t src_batch_stride, void* dst,
                            int64_t dst_row_stride, int64_t dst_batch_stride, int B, int rows, int row_bytes,
                            hipStream_t stream) {
    if (B == 0 || rows == 0 || row_bytes == 0) return hipSuccess;
    const int row_words = row_bytes / 16;
    const long total = (long)rows * row_words;
    const unsigned bx = (unsigned)std::min<long>((total + 255) / 256, 1024);
    hipLaunchKernelGGL(copy_rows_kernel, dim3(bx, B), dim3(256), 0, stream, static_cast<const char*>(src),
                       src_row_stride, src_batch_stride, static_cast<char*>(dst), dst_row_stride, dst_batch_stride,
                       rows, row_words);
    return hipGetLastError();
}

}  // namespace ssd
