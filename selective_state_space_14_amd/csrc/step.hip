// step.hip -- ssd_step: one decode token per sequence on gfx950.
//
// Per sequence b (one workgroup of 1024 threads):
//   1. conv window [conv_state rows 0..K-2, new raw row] -> act -> rounded to
//      the storage dtype (as a prefill would store it) -> fp32 in LDS; the
//      conv buffer shifts by one row in place (same thread reads then writes
//      each channel, so no other thread can observe a half-shifted buffer);
//      dt = softplus(dt_raw + dt_bias) and a = exp(dt * A) per head in LDS.
//   2. a streaming read-modify-write of the fp32 state [H][P][N]: each thread
//      owns one float4 (4 consecutive n of one p row) per item;
//          h[p, n] = a * h[p, n] + (dt * x_p) * B_n
//      and the N/4 lanes of a row reduce C . h with a fixed xor butterfly,
//      so the result is deterministic and independent of the batch size.
//   y[p] = (C . h[p] + D x_p) * silu(z_p).
// The state is 96% of the bytes (B*H*P*N*4 read + written per token).  Items
// are processed kStepUnroll at a time with the next batch's loads issued
// before the current batch is computed (the first batch even before the conv
// phase), so each thread keeps up to 128 B of state in flight; the item index
// decodes into (head, p, n-quad) with shifts (P = 64, N a power of two).
// The recurrence is the Mamba-2 SSD layer of the Codestral-Mamba port header
// (codestral_mamba.ts); step == forward at length 1 with the state carried
// follows mojolearn.Mamba3Block's step() description.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kStepThreads = 1024;
constexpr int kStepUnroll = 4;
constexpr int kP = 64;             // head dim (the only one the library accepts)

template <typename T> struct Vec16;
template <> struct Vec16<float> { static constexpr int n = 4; };
template <> struct Vec16<uint16_t> { static constexpr int n = 8; };

// 16 bytes of T values -> VEC fp32 values.
__device__ __forceinline__ void unpack16(uint4 v, float* out, float*) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(uint4 v, float* out, uint16_t*) {
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x); out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z); out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
}
__device__ __forceinline__ float round_to(float v, float*) { return v; }
__device__ __forceinline__ float round_to(float v, uint16_t*) { return __uint_as_float(f32_to_bf16_bits(v) << 16); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T, int N>
__global__ __launch_bounds__(kStepThreads) void ssd_step_kernel(StepArgs a) {
    extern __shared__ float smem[];
    constexpr int VEC = Vec16<T>::n;
    constexpr int K = 4;
    constexpr int P = kP;
    const int H = a.H, G = a.G;
    const int HP = H * P, GN = G * N, C = HP + 2 * GN;
    const int hpg = H / G;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    float* xbc_s = smem;              // [C]
    float* dt_s = smem + C;           // [H]
    float* a_s = dt_s + H;            // [H]
    int* gofs_s = reinterpret_cast<int*>(a_s + H);   // [H]: offset of the head's group in B and C

    // state items: float4 f of this sequence is (h, p, n-quad) = (f / (P NQ), (f / NQ) % P, f % NQ)
    constexpr int NQ = N / 4;                       // lanes per p row
    constexpr int per_head = P * NQ;                // float4 items per head (a power of two)
    const int total = H * per_head;
    float4* st = reinterpret_cast<float4*>(a.ssm_state + (size_t)b * H * P * N);
    float4 s_cur[kStepUnroll], s_nxt[kStepUnroll];
    auto load_batch = [&](int base, float4* dst) {
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) {
            const int f = base + u * kStepThreads + tid;
            dst[u] = f < total ? st[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    load_batch(0, s_cur);             // independent of the conv phase: start it now

    // ---- 1. conv window, activation, buffer shift
    const T* raw = static_cast<const T*>(a.xbc_raw) + (size_t)b * C;
    T* cst = static_cast<T*>(a.conv_state) + (size_t)b * (K - 1) * C;
    for (int c0 = tid * VEC; c0 < C; c0 += kStepThreads * VEC) {
        // the three carried rows and the new row, as raw 16-byte words
        const uint4 q0 = *reinterpret_cast<const uint4*>(cst + c0);
        const uint4 q1 = *reinterpret_cast<const uint4*>(cst + C + c0);
        const uint4 q2 = *reinterpret_cast<const uint4*>(cst + 2 * C + c0);
        const uint4 qr = *reinterpret_cast<const uint4*>(raw + c0);
        // shift: row0 <- row1, row1 <- row2, row2 <- new row (bits copied as they are)
        *reinterpret_cast<uint4*>(cst + c0) = q1;
        *reinterpret_cast<uint4*>(cst + C + c0) = q2;
        *reinterpret_cast<uint4*>(cst + 2 * C + c0) = qr;
        float r0[VEC], r1[VEC], r2[VEC], cur[VEC];
        unpack16(q0, r0, (T*)nullptr);
        unpack16(q1, r1, (T*)nullptr);
        unpack16(q2, r2, (T*)nullptr);
        unpack16(qr, cur, (T*)nullptr);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int c = c0 + e;
            float4 w = *reinterpret_cast<const float4*>(a.conv_w + (size_t)c * K);
            float v = a.conv_b ? a.conv_b[c] : 0.0f;
            v = fmaf(w.x, r0[e], v);
            v = fmaf(w.y, r1[e], v);
            v = fmaf(w.z, r2[e], v);
            v = fmaf(w.w, cur[e], v);
            if (a.act == 0) v = silu_f(v);
            xbc_s[c] = round_to(v, (T*)nullptr);
        }
    }
    for (int h = tid; h < H; h += kStepThreads) {
        float r = load1(static_cast<const T*>(a.dt_raw) + (size_t)b * H + h);
        float dt = softplus_f(r + (a.dt_bias ? a.dt_bias[h] : 0.0f));
        dt_s[h] = dt;
        a_s[h] = expf(dt * a.A[h]);
        gofs_s[h] = (h / hpg) * N;
    }
    __syncthreads();

    // ---- 2. state read-modify-write
    const T* zb = a.z ? static_cast<const T*>(a.z) + (size_t)b * HP : nullptr;
    float* yb = a.y + (size_t)b * HP;
    constexpr int kBatchItems = kStepThreads * kStepUnroll;
    for (int base = 0; base < total; base += kBatchItems) {
        if (base + kBatchItems < total) load_batch(base + kBatchItems, s_nxt);
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) {
            const int f = base + u * kStepThreads + tid;
            const bool live = f < total;
            // a wave's 64 items lie in one head (per_head and total are multiples of 64)
            const int h = __builtin_amdgcn_readfirstlane(min(f, total - 1) / per_head);
            const int p = (f / NQ) % P;
            const int nq = f % NQ;
            const int gofs = gofs_s[h];
            const float dt = dt_s[h], dec = a_s[h];
            const float xp = xbc_s[h * P + p];
            const float dx = dt * xp;
            const float4 Bv = *reinterpret_cast<const float4*>(xbc_s + HP + gofs + 4 * nq);
            const float4 Cv = *reinterpret_cast<const float4*>(xbc_s + HP + GN + gofs + 4 * nq);
            float4 v = s_cur[u];
            v.x = fmaf(dec, v.x, dx * Bv.x);
            v.y = fmaf(dec, v.y, dx * Bv.y);
            v.z = fmaf(dec, v.z, dx * Bv.z);
            v.w = fmaf(dec, v.w, dx * Bv.w);
            float part = Cv.x * v.x;
            part = fmaf(Cv.y, v.y, part);
            part = fmaf(Cv.z, v.z, part);
            part = fmaf(Cv.w, v.w, part);
#pragma unroll
            for (int off = 1; off < NQ; off <<= 1) part += __shfl_xor(part, off, NQ);
            if (live) {
                st[f] = v;
                if (nq == 0) {
                    float yv = part + (a.D ? a.D[h] : 0.0f) * xp;
                    if (zb) yv *= silu_f(load1(zb + h * P + p));
                    yb[h * P + p] = yv;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) s_cur[u] = s_nxt[u];
    }
}

template <typename T, int N>
hipError_t launch_step_n(const StepArgs& a, hipStream_t stream) {
    const int C = a.H * a.P + 2 * a.G * N;
    const size_t lds = sizeof(float) * ((size_t)C + 3 * a.H);
    hipLaunchKernelGGL((ssd_step_kernel<T, N>), dim3(a.B), dim3(kStepThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_step_t(const StepArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_step_n<T, 16>(a, stream);
        case 32: return launch_step_n<T, 32>(a, stream);
        case 64: return launch_step_n<T, 64>(a, stream);
        case 128: return launch_step_n<T, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t step_lds_bytes(int H, int P, int N, int G) {
    return sizeof(float) * ((size_t)H * P + 2 * (size_t)G * N + 3 * (size_t)H);
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 0 ? launch_step_t<float>(a, stream) : launch_step_t<uint16_t>(a, stream);
}

}  // namespace ssd
