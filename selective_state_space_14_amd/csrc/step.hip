// step.hip -- ssd_step: one decode token per sequence on gfx950.
//
// Per sequence b (one workgroup of 1024 threads):
//   1. the B and C columns: conv window [conv_state rows 0..K-2, new raw
//      row] -> act -> rounded to the storage dtype (as a prefill would store
//      it) -> fp32 in LDS, the conv buffer shifting by one row in place (the
//      thread that reads a channel's rows writes them); dt = softplus(dt_raw +
//      dt_bias) and a = exp(dt * A) per head in LDS.
//   2. a streaming read-modify-write of the fp32 state [H][P][N], a round of
//      rows at a time: eight lanes share a row (four float4 each for N = 128);
//      row h*P + p also convolves x channel h*P + p (its inputs loaded one
//      round ahead) and shifts that channel's buffer rows, then
//          h[p, n] = a * h[p, n] + (dt * x_p) * B_n
//      and the row's lanes reduce C . h with a fixed DPP butterfly, so the
//      result is deterministic and independent of the batch size;
//   y[p] = (C . h[p] + D x_p) * silu(z_p).
// The state is 96% of the bytes (B*H*P*N*4 read + written per token): its
// loads and stores are nontemporal (it is touched once per token), loads run
// one round ahead of the round being computed (deeper prefetch measured no
// faster: 64 KB per round and CU already covers the latency), and the first
// round's loads are issued even before the B/C conv phase.
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
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }

typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Sum over aligned groups of W lanes (W = 4 or 8), every lane of a group
// receiving the group's sum: quad-permute xor 1, xor 2, then (W = 8) the
// half-row mirror, which pairs each lane with one of the other quad.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int W>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(W == 4 || W == 8, "group width");
    v = dpp_add<0xB1>(v);            // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);            // quad_perm [2,3,0,1]
    if (W == 8) v = dpp_add<0x141>(v);   // row_half_mirror
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
    float* xbc_s = smem;              // [C]
    float* dt_s = smem + C;           // [H]
    float* a_s = dt_s + H;            // [H]
    int* gofs_s = reinterpret_cast<int*>(a_s + H);   // [H]: offset of the head's group in B and C
    float* d_s = a_s + 2 * H;                         // [H]: D (0 when absent)

    // ---- state rows: row = h * P + p holds NQ float4 (n fastest).  LPR lanes
    // share a row, lane q of a row holds float4 q + LPR j (j < FPL), so every
    // load instruction reads whole 128-byte row segments; a wave covers RPW
    // consecutive rows (one head) per round, the workgroup RPR rows.
    constexpr int NQ = N / 4;
    constexpr int LPR = NQ < 8 ? NQ : 8;
    constexpr int FPL = NQ / LPR;
    constexpr int RPW = 64 / LPR;
    constexpr int RPR = RPW * (kStepThreads / 64);
    const int nrows = H * P;                         // a multiple of 64, so rounds cover whole waves
    const int wave = tid >> 6, lane = tid & 63;
    const int q = lane % LPR;
    // The state goes through range-checked buffer loads and stores with the
    // nontemporal bit: rows past the end read 0 and their stores are dropped,
    // so the loop has no branches around memory operations and the compiler
    // counts the loads in flight exactly.
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        a.ssm_state + (size_t)b * H * P * N, 0, nrows * NQ * 16, 0x00020000);
    constexpr int kNT = 2;                           // cache policy: nontemporal
    f4v s_cur[FPL], s_nxt[FPL];       // rounds r, r+1
    auto row_of = [&](int r) { return r * RPR + wave * RPW + lane / LPR; };
    auto off_of = [&](int row, int j) { return (uint32_t)((row * NQ + q + j * LPR) * 16); };
    auto load_round = [&](int r, f4v* dst) {
        const int row = row_of(r);
#pragma unroll
        for (int j = 0; j < FPL; ++j)
            dst[j] = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(sr, off_of(row, j), 0, kNT));
    };
    load_round(0, s_cur);             // independent of the conv phase: start it now

    // ---- 1. the B and C columns: conv window, activation, buffer shift, to
    // LDS (every state row reads them); dt, the decay, D per head.  The x
    // columns are convolved inside the state loop by the rows they feed.
    const T* raw = static_cast<const T*>(a.xbc_raw) + (size_t)b * C;
    T* cst = static_cast<T*>(a.conv_state) + (size_t)b * (K - 1) * C;
    for (int c0 = HP + tid * VEC; c0 < C; c0 += kStepThreads * VEC) {
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
            const float4 w = *reinterpret_cast<const float4*>(a.conv_w + (size_t)c * K);
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
        d_s[h] = a.D ? a.D[h] : 0.0f;
    }

    // ---- per-row x inputs, loaded one round ahead of their use: row h*P + p
    // is x channel h*P + p, so a row's lanes convolve their own channel (all
    // of them, from the same addresses) and its first lane shifts the buffer.
    const T* zb = a.z ? static_cast<const T*>(a.z) + (size_t)b * HP : nullptr;
    struct XIn {
        T q0, q1, q2, qr;     // carried rows and the new raw value (bits as stored)
        float4 w;
        float bias, z;
    };
    auto load_x = [&](int r, XIn& o) {
        const int ch = min(row_of(r), nrows - 1);    // the row's x channel, clamped past the end
        o.q0 = cst[ch];
        o.q1 = cst[C + ch];
        o.q2 = cst[2 * C + ch];
        o.qr = raw[ch];
        o.w = *reinterpret_cast<const float4*>(a.conv_w + (size_t)ch * K);
        o.bias = a.conv_b ? a.conv_b[ch] : 0.0f;
        o.z = zb ? load1(zb + ch) : 0.0f;
    };
    XIn x_cur, x_nxt;
    load_x(0, x_cur);
    __syncthreads();

    // ---- 2. state read-modify-write, one round of RPR rows at a time; the
    // next round's loads are issued before the current round is computed
    // y through a range-checked buffer store: lanes other than a row's first
    // aim past the range and are dropped, so the store is never skipped
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)b * HP, 0, HP * 4, 0x00020000);
    const int nrounds = (nrows + RPR - 1) / RPR;
    // B and C of this lane's n-quads for the current group, reloaded only when
    // the group changes (never, for one group)
    float4 Bq[FPL], Cq[FPL];
    int cur_gofs = -1;
    for (int r = 0; r < nrounds; ++r) {
        load_round(r + 1, s_nxt);                    // past the last round: out of range, reads 0
        load_x(r + 1, x_nxt);
        const int row = row_of(r);
        // a wave's rows lie in one head; a wave past the end computes on clamped
        // rows and its stores fall outside the ranges or are skipped
        const int hrow = min(row, nrows - 1);
        const int h = __builtin_amdgcn_readfirstlane(hrow / P);
        const int p = hrow % P;
        const int gofs = gofs_s[h];
        if (gofs != cur_gofs) {                     // uniform: gofs is per head
            cur_gofs = gofs;
#pragma unroll
            for (int j = 0; j < FPL; ++j) {
                Bq[j] = *reinterpret_cast<const float4*>(xbc_s + HP + gofs + 4 * (q + j * LPR));
                Cq[j] = *reinterpret_cast<const float4*>(xbc_s + HP + GN + gofs + 4 * (q + j * LPR));
            }
        }
        // the row's x channel: conv window, activation, rounded to T as a prefill stores it
        float xp;
        {
            float v = x_cur.bias;
            v = fmaf(x_cur.w.x, to_f32(x_cur.q0), v);
            v = fmaf(x_cur.w.y, to_f32(x_cur.q1), v);
            v = fmaf(x_cur.w.z, to_f32(x_cur.q2), v);
            v = fmaf(x_cur.w.w, to_f32(x_cur.qr), v);
            if (a.act == 0) v = silu_f(v);
            xp = round_to(v, (T*)nullptr);
        }
        if (q == 0 && row < nrows) {                 // shift the channel's buffer rows
            cst[row] = x_cur.q1;
            cst[C + row] = x_cur.q2;
            cst[2 * C + row] = x_cur.qr;
        }
        const float dec = a_s[h];
        const float dx = dt_s[h] * xp;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < FPL; ++j) {
            const float4 Bv = Bq[j], Cv = Cq[j];
            f4v v = s_cur[j];
            v.x = fmaf(dec, v.x, dx * Bv.x);
            v.y = fmaf(dec, v.y, dx * Bv.y);
            v.z = fmaf(dec, v.z, dx * Bv.z);
            v.w = fmaf(dec, v.w, dx * Bv.w);
            part = fmaf(Cv.x, v.x, part);
            part = fmaf(Cv.y, v.y, part);
            part = fmaf(Cv.z, v.z, part);
            part = fmaf(Cv.w, v.w, part);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sr, off_of(row, j), 0, kNT);
        }
        // sum over the LPR lanes of the row (a fixed order: deterministic)
        part = row_sum<LPR>(part);
        float yv = fmaf(d_s[h], xp, part);
        if (zb) yv *= silu_f(x_cur.z);
        const bool first = q == 0 && row < nrows;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yr, first ? (uint32_t)(h * P + p) * 4 : 0x7fffffffu, 0, 0);
#pragma unroll
        for (int j = 0; j < FPL; ++j) {
            s_cur[j] = s_nxt[j];
        }
        x_cur = x_nxt;
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
