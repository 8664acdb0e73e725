// step.hip -- ssd_step: one decode token per sequence on gfx950.
//
// Per sequence b (one workgroup of 1024 threads):
//   1. every conv channel: window [conv_state rows 0..K-2, new raw row] ->
//      act -> rounded to the storage dtype (as a prefill would store it) ->
//      fp32 in LDS, the conv buffer shifting by one row in place (the thread
//      that reads a channel's rows writes them); silu(z), dt = softplus(dt_raw
//      + dt_bias) and a = exp(dt * A) per head, in LDS too.
//   2. a streaming read-modify-write of the fp32 state [H][P][N], a round of
//      64 KiB at a time, thread t holding float4 t + 1024 j of the round, so
//      each instruction of the workgroup covers 16 KiB of contiguous state;
//          h[p, n] = a * h[p, n] + (dt * x_p) * B_n
//      and the N/4 lanes of a row reduce C . h with a fixed butterfly, so the
//      result is deterministic and independent of the batch size;
//   y[p] = (C . h[p] + D x_p) * silu(z_p).
// The state is 96% of the bytes (B*H*P*N*4 read + written per token): its
// loads and stores are nontemporal (it is touched once per token), loads run
// one round ahead of the round being computed, and the first round's loads
// are issued before the conv phase.
// The recurrence is the Mamba-2 SSD layer of the Codestral-Mamba port header
// (codestral_mamba.ts); step == forward at length 1 with the state carried
// follows mojolearn.Mamba3Block's step() description.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kStepThreads = 1024;
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

typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Sum over aligned groups of W consecutive lanes (W = 4, 8, 16 or 32) in a
// fixed butterfly: quad permutes xor 1 and xor 2, then the half-row mirror
// (lane i with 7 - i) and the row mirror (i with 15 - i), after each of which
// the partners hold equal partial sums; for W = 32 the row broadcast then adds
// lane 15 of each even 16-lane row into the odd row after it.  The group's
// last lane always holds the group's sum, and the order of every addition is
// fixed, so the result does not depend on the batch.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "group width");
    v = dpp_add<0xB1>(v);                 // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);                 // quad_perm [2,3,0,1]
    if (W >= 8) v = dpp_add<0x141>(v);    // row_half_mirror
    if (W >= 16) v = dpp_add<0x140>(v);   // row_mirror
    if (W >= 32) v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));   // row_bcast:15
    return v;
}

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
    float* xz_s = smem;               // [H*P][2]: per x channel, the convolved x and its gate silu(z) (1 without z)
    float* bc_s = smem + 2 * HP;      // [2*G*N]: the convolved B columns, then the C columns
    float4* hd_s = reinterpret_cast<float4*>(bc_s + 2 * GN);   // [H]: per head {exp(dt A), dt, D (0 when absent), 0}

    // ---- the state [H*P rows][N] as a flat array of float4: round r covers
    // float4 r*4096 .. +4095, and thread t holds float4 t + 1024 j of it (j <
    // F).  Each load or store instruction of the workgroup therefore covers
    // 16 KiB of contiguous state (measured here at ~6.2 TB/s for this
    // read-modify-write, against ~5.5 TB/s when each wave instead streams its
    // own 4 KiB).  A row's NQ float4 sit in NQ consecutive lanes; the lane's
    // n-quad q = t mod NQ is the same in every round.
    constexpr int NQ = N / 4;
    constexpr int F = 4;
    constexpr int PER_ROUND = kStepThreads * F;
    const int nrows = HP;
    const int total = nrows * NQ;
    const int nrounds = (total + PER_ROUND - 1) / PER_ROUND;
    const int q = tid % NQ;
    // range-checked nontemporal buffer operations: float4 past the end read 0
    // and their stores are dropped, so no memory operation sits under a branch
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        a.ssm_state + (size_t)b * H * P * N, 0, total * 16, 0x00020000);
    constexpr int kNT = 2;                           // cache policy: nontemporal
    auto idx = [&](int r, int j) { return r * PER_ROUND + j * kStepThreads + tid; };
    f4v s_cur[F], s_nxt[F];           // rounds r, r+1
    auto load_round = [&](int r, f4v* dst) {
#pragma unroll
        for (int j = 0; j < F; ++j)
            dst[j] = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(sr, (uint32_t)idx(r, j) * 16u, 0, kNT));
    };
    load_round(0, s_cur);             // independent of the conv phase: start it now

    // ---- 1. every conv channel up front: window [conv_state rows 0..K-2, new
    // raw row] -> act -> rounded to the storage dtype (as a prefill would store
    // it) -> fp32 in LDS, the buffer shifting by one row in place (the thread
    // that reads a channel's rows writes them); silu(z) of the x channels;
    // dt = softplus(dt_raw + dt_bias) and a = exp(dt * A) per head.
    const T* raw = static_cast<const T*>(a.xbc_raw) + (size_t)b * C;
    T* cst = static_cast<T*>(a.conv_state) + (size_t)b * (K - 1) * C;
    const T* zb = a.z ? static_cast<const T*>(a.z) + (size_t)b * HP : nullptr;
    // the gate inputs first: the conv loop below stores, and these loads must not wait behind it
    constexpr int ZI = 4096 / (kStepThreads * VEC) > 0 ? 4096 / (kStepThreads * VEC) : 1;
    uint4 zq[ZI];
#pragma unroll
    for (int i = 0; i < ZI; ++i) {
        const int c0 = (tid + i * kStepThreads) * VEC;
        zq[i] = zb && c0 < HP ? *reinterpret_cast<const uint4*>(zb + c0) : make_uint4(0, 0, 0, 0);
    }
    // per-head inputs, one head per thread (the LDS budget keeps H*P, so H, far below 1024)
    float dt_in = 0.0f, A_h = 0.0f, D_h = 0.0f;
    if (tid < H) {
        dt_in = load1(static_cast<const T*>(a.dt_raw) + (size_t)b * H + tid) + (a.dt_bias ? a.dt_bias[tid] : 0.0f);
        A_h = a.A[tid];
        D_h = a.D ? a.D[tid] : 0.0f;
    }
    // one conv group: VEC channels from c0, their three carried rows and new
    // row as raw 16-byte words; the rows shift by one (row0 <- row1, row1 <-
    // row2, row2 <- new row, bits copied as they are) and the convolved,
    // activated, storage-rounded values go to LDS
    auto conv_group = [&](int c0, const uint4 (&w)[4]) {
        *reinterpret_cast<uint4*>(cst + c0) = w[1];
        *reinterpret_cast<uint4*>(cst + C + c0) = w[2];
        *reinterpret_cast<uint4*>(cst + 2 * C + c0) = w[3];
        float r0[VEC], r1[VEC], r2[VEC], cur[VEC];
        unpack16(w[0], r0, (T*)nullptr);
        unpack16(w[1], r1, (T*)nullptr);
        unpack16(w[2], r2, (T*)nullptr);
        unpack16(w[3], cur, (T*)nullptr);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int c = c0 + e;
            const float4 cw = *reinterpret_cast<const float4*>(a.conv_w + (size_t)c * K);
            float v = a.conv_b ? a.conv_b[c] : 0.0f;
            v = fmaf(cw.x, r0[e], v);
            v = fmaf(cw.y, r1[e], v);
            v = fmaf(cw.z, r2[e], v);
            v = fmaf(cw.w, cur[e], v);
            if (a.act == 0) v = silu_f(v);
            v = round_to(v, (T*)nullptr);
            if (c < HP) xz_s[2 * c] = v;
            else bc_s[c - HP] = v;
        }
    };
    auto conv_load = [&](int c0, uint4 (&w)[4]) {
        w[0] = *reinterpret_cast<const uint4*>(cst + c0);
        w[1] = *reinterpret_cast<const uint4*>(cst + C + c0);
        w[2] = *reinterpret_cast<const uint4*>(cst + 2 * C + c0);
        w[3] = *reinterpret_cast<const uint4*>(raw + c0);
    };
    // the first two groups of every thread load before either stores, so a
    // thread with two groups waits for one memory latency, not two
    constexpr int CI = 2;
    uint4 cw_in[CI][4];
#pragma unroll
    for (int i = 0; i < CI; ++i) {
        const int c0 = (tid + i * kStepThreads) * VEC;
        if (c0 < C) conv_load(c0, cw_in[i]);
    }
#pragma unroll
    for (int i = 0; i < CI; ++i) {
        const int c0 = (tid + i * kStepThreads) * VEC;
        if (c0 < C) conv_group(c0, cw_in[i]);
    }
    for (int c0 = (tid + CI * kStepThreads) * VEC; c0 < C; c0 += kStepThreads * VEC) {
        uint4 w[4];
        conv_load(c0, w);
        conv_group(c0, w);
    }
    if (tid < H) {
        const float dt = softplus_f(dt_in);
        hd_s[tid] = make_float4(expf(dt * A_h), dt, D_h, 0.0f);
    }
#pragma unroll
    for (int i = 0; i < ZI; ++i) {
        const int c0 = (tid + i * kStepThreads) * VEC;
        if (c0 < HP) {
            float zz[VEC];
            unpack16(zq[i], zz, (T*)nullptr);
#pragma unroll
            for (int e = 0; e < VEC; ++e) xz_s[2 * (c0 + e) + 1] = zb ? silu_f(zz[e]) : 1.0f;
        }
    }
    for (int c0 = (tid + ZI * kStepThreads) * VEC; c0 < HP; c0 += kStepThreads * VEC) {
        float zz[VEC];
        if (zb) unpack16(*reinterpret_cast<const uint4*>(zb + c0), zz, (T*)nullptr);
#pragma unroll
        for (int e = 0; e < VEC; ++e) xz_s[2 * (c0 + e) + 1] = zb ? silu_f(zz[e]) : 1.0f;
    }
    __syncthreads();

    // ---- 2. state read-modify-write, one round at a time, the next round's
    // loads issued before the current round is computed:
    //     h[p, n] = a * h[p, n] + (dt * x_p) * B_n,   y[p] = (C . h[p] + D x_p) * silu(z_p)
    // y through a range-checked buffer store: lanes other than a row's last
    // aim past the range and are dropped, so the store is never skipped
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)b * HP, 0, HP * 4, 0x00020000);
    // h / hpg as a multiply and shift: with m = floor((2^32 - 1) / hpg) + 1
    // (2^32 for hpg = 1), h * m / 2^32 exceeds h / hpg by less than h / 2^32,
    // which stays below the gap 1 / hpg to the next integer while h * hpg < 2^32
    // (here h < H <= 2^16)
    const uint64_t inv_hpg = 0xffffffffull / (uint64_t)hpg + 1ull;
    for (int r = 0; r < nrounds; ++r) {
        load_round(r + 1, s_nxt);                    // past the last round: out of range, reads 0
        // every LDS operand of the round first, so their latencies overlap
        int f[F], row[F];
        float2 xz[F];                 // x_p, silu(z_p)
        float4 hd[F], Bv[F], Cv[F];   // {a, dt, D, 0} of the head; B and C of its group
#pragma unroll
        for (int j = 0; j < F; ++j) {
            f[j] = idx(r, j);
            row[j] = f[j] < total ? f[j] / NQ : nrows - 1;   // past the end: the last row, nothing kept
            // a wave's 64 float4 are 64-aligned and a head's P*N/4 (>= 256)
            // float4 start at a multiple of 64: the head is the wave's
            const int h = __builtin_amdgcn_readfirstlane(row[j] / P);
            const int gofs = (int)(((uint64_t)(uint32_t)h * inv_hpg) >> 32) * N;
            xz[j] = *reinterpret_cast<const float2*>(xz_s + 2 * row[j]);
            hd[j] = hd_s[h];
            Bv[j] = *reinterpret_cast<const float4*>(bc_s + gofs + 4 * q);
            Cv[j] = *reinterpret_cast<const float4*>(bc_s + GN + gofs + 4 * q);
        }
        float part[F];
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const float dxj = hd[j].y * xz[j].x;
            const float dec = hd[j].x;
            f4v v = s_cur[j];
            v.x = fmaf(dec, v.x, dxj * Bv[j].x);
            v.y = fmaf(dec, v.y, dxj * Bv[j].y);
            v.z = fmaf(dec, v.z, dxj * Bv[j].z);
            v.w = fmaf(dec, v.w, dxj * Bv[j].w);
            float s = Cv[j].x * v.x;
            s = fmaf(Cv[j].y, v.y, s);
            s = fmaf(Cv[j].z, v.z, s);
            part[j] = fmaf(Cv[j].w, v.w, s);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sr, (uint32_t)f[j] * 16u, 0, kNT);
        }
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const float yv = fmaf(hd[j].z, xz[j].x, group_sum<NQ>(part[j])) * xz[j].y;
            const bool first = q == NQ - 1 && f[j] < total;   // the group's last lane holds its sum
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yr, first ? (uint32_t)row[j] * 4 : 0x7fffffffu, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < F; ++j) s_cur[j] = s_nxt[j];
    }
}

template <typename T, int N>
hipError_t launch_step_n(const StepArgs& a, hipStream_t stream) {
    const int C = a.H * a.P + 2 * a.G * N;
    const size_t lds = sizeof(float) * ((size_t)C + 4 * a.H + (size_t)a.H * a.P);
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
    return sizeof(float) * (2 * (size_t)H * P + 2 * (size_t)G * N + 4 * (size_t)H);
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 0 ? launch_step_t<float>(a, stream) : launch_step_t<uint16_t>(a, stream);
}

}  // namespace ssd
