// s6.hip -- ssd_s6_scan_fwd: the Mamba-1 selective scan (S6) on gfx950.
//
// Per batch row b and channel d, with a diagonal state of N entries:
//     h_t[n] = exp(dt_t A[d][n]) h_{t-1}[n] + dt_t B_t[n] x_t
//     y_t    = (sum_n C_t[n] h_t[n] + D[d] x_t) silu(z_t)
// (falcon_mamba.ts header: x_proj rows [dt, B, C] give one B and one C per
// token for every channel; dt comes from dt_proj with its bias inside the
// softplus; A [d_inner, d_state] = -exp(A_log).)  Unlike the SSD scan the
// decay differs per (d, n), so there is no low-rank chunk form for MFMA: the
// recurrence runs token by token, one channel per lane with its N states and
// N decay rates in registers.  B_t and C_t are the same for every lane of a
// token: they are staged once per tile in LDS (as fp32) and read by broadcast.
// Per token and channel the work is N exp2 and ~4N other VALU instructions,
// against 10 bytes of HBM traffic (bf16 x, dt, z in, fp32 y out), so the
// kernel is bound by the VALU, not by HBM.
//
// Parallelism: B * D lanes are too few waves for the chip, so the sequence is
// cut into K superchunks as in the SSD scan: a state-only pre-pass stores each
// superchunk's local end state and sum of dt (its decay is exp(A sum dt) per
// (d, n), or a reset marker when a document starts inside it), and the main
// pass folds the preceding ones into its starting state.
#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kS6Threads = 256;                    // one channel per thread
constexpr int kS6TileBf16 = 16, kS6TileF32 = 8;    // tokens per LDS tile
constexpr bool kS6Pipe = false;                    // true: the next token's reads overlap this token's update
constexpr long kS6WgPerCu = 3;                     // resident workgroups per CU the split aims at
constexpr float kLn2 = 0.6931471805599453f;
enum { kS6Full = 0, kS6State = 1 };
typedef unsigned s6_u32x4 __attribute__((ext_vector_type(4)));

// softplus(v) = max(v, 0) + log(1 + e^-|v|) on the hardware exp2 / log2: a few
// ulp, except that softplus of v below about -17 (under 2^-24) reads as 0.
__device__ __forceinline__ float softplus_hw(float v) {
    return fmaxf(v, 0.0f) + __builtin_amdgcn_logf(1.0f + fast_exp2(-fabsf(v) * kLog2e)) * kLn2;
}

__device__ __forceinline__ float s6_ld(const float* p) { return *p; }
__device__ __forceinline__ float s6_ld(const uint16_t* p) { return bf16_to_f32(*p); }

// n values of a row that every lane reads (LDS broadcast)
template <int n> __device__ __forceinline__ void s6_row(const float* p, float* out) {
#pragma unroll
    for (int i = 0; i < n; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + i);
        out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
    }
}

// A range-checked buffer over a [rows][stride] tensor from element `first`
// on: reads past the tensor's last element return 0 instead of faulting.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t s6_rsrc(const void* base, size_t first, size_t total) {
    const size_t left = total > first ? (total - first) * sizeof(T) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(static_cast<const T*>(base)) + first, 0,
                                             (int)(left < 0x7fffffffu ? left : 0x7fffffffu), 0x00020000);
}

// Tiles of TT tokens: x, dt (and z) for the workgroup's 256 channels and the
// B (and C) rows are staged in LDS by 16-byte loads, the next tile's loads
// in flight (in registers) while the current tile is scanned.
template <typename T, int N, int MODE>
struct S6Tile {
    static constexpr int TT = sizeof(T) == 2 ? kS6TileBf16 : kS6TileF32;
    static constexpr int ROWB = kS6Threads * (int)sizeof(T);            // bytes of one token's channels
    static constexpr int PPT = TT * ROWB / 16 / kS6Threads;             // 16-byte pieces per thread per tensor
    static constexpr int NT = MODE == kS6Full ? 3 : 2;                  // x, dt (, z)
    static constexpr int BCB = TT * N * (int)sizeof(T);                 // bytes of a tile of B rows
    static constexpr int BCP = BCB / 16;                                // its 16-byte pieces
    static_assert(PPT >= 1 && TT * ROWB == PPT * 16 * kS6Threads, "tile");
    static_assert(2 * BCP <= kS6Threads && BCB % 16 == 0, "B/C pieces");
};

template <typename T, int N, int MODE>
__global__ __launch_bounds__(kS6Threads) void ssd_s6_kernel(S6Args a) {
    constexpr bool FULL = MODE == kS6Full;
    using TL = S6Tile<T, N, MODE>;
    constexpr int TT = TL::TT, PPT = TL::PPT, NT = TL::NT, BCP = TL::BCP;
    __shared__ __attribute__((aligned(16))) T s_act[NT][TT][kS6Threads];   // x, dt, z
    __shared__ __attribute__((aligned(16))) float s_bc[2][TT][N];         // B, C rows (fp32)
    __shared__ uint32_t s_mask;                                          // document starts in the tile

    const int D = a.D, L = a.L;
    const int tid = threadIdx.x;
    const int nblk = (D + kS6Threads - 1) / kS6Threads;
    const int KU = FULL ? a.K : a.K - 1;
    const int id = blockIdx.x;
    const int blk = id % nblk;
    const int k = (id / nblk) % KU;
    const int b = id / (nblk * KU);
    const int c0 = blk * kS6Threads;
    const int d = c0 + tid;
    const bool on = d < D;
    const int dc = min(d, D - 1);                  // lanes past D compute on the last channel, store nothing
    const int tbeg = k * a.S;
    const int tend = min(tbeg + a.S, L);

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[(size_t)dc * N + n] * kLog2e;
        h[n] = 0.0f;
    }
    const float bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    const float Dd = a.D_skip ? a.D_skip[dc] : 0.0f;
    const size_t sidx = (size_t)b * D + dc;        // channel index for the states

    if (FULL) {
        // the given initial state (the pre-pass's copy under the split), then
        // the superchunks before k folded in order
        const float* h_init = a.K > 1 ? a.h0 : a.init_state;
        if (h_init) {
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = h_init[sidx * N + n];
        }
        for (int j = 0; j < k; ++j) {
            const size_t u = sidx * (a.K - 1) + j;
            const float sdt = a.sdt[u];
            const float* hl = a.hloc + u * N;
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = sdt == -INFINITY ? hl[n] : fmaf(fast_exp2(A2[n] * sdt), h[n], hl[n]);
        }
    } else if (k == 0 && a.h0 && on) {
        // the main pass reads this copy instead of init_state
#pragma unroll
        for (int n = 0; n < N; ++n) a.h0[sidx * N + n] = a.init_state[sidx * N + n];
    }

    // ---- staging: 16-byte pieces of the [TT][256] activation tiles and of the
    // [TT][N] B / C tiles, through range-checked buffer loads
    const size_t rows = (size_t)a.B * L;
    const bool has_z = FULL && a.z != nullptr;
    const void* act_src[3] = {a.x, a.dt, a.z};
    const int64_t act_stride[3] = {a.x_stride, a.dt_stride, a.z_stride};
    const int bcsel = tid < BCP ? 0 : 1;           // threads [0, BCP) load B, [BCP, 2 BCP) C
    const int bcp = tid - bcsel * BCP;
    const bool bc_on = tid < 2 * BCP && (FULL || bcsel == 0);
    const void* bc_src = bcsel ? a.Cm : a.Bm;
    const int64_t bc_stride = bcsel ? a.C_stride : a.B_stride;
    constexpr int PPR_BC = N * (int)sizeof(T) / 16;    // pieces of one B row
    const int32_t* doc = a.doc ? a.doc + (size_t)b * L : nullptr;

    s6_u32x4 r_act[NT][PPT], r_bc;
    int r_doc0 = 0, r_doc1 = 0;
    auto issue = [&](int t0) {
        const size_t row0 = (size_t)b * L + t0;
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            if (q == 2 && !has_z) break;
            const __amdgpu_buffer_rsrc_t rs = s6_rsrc<T>(act_src[q], row0 * act_stride[q] + c0,
                                                         (rows - 1) * act_stride[q] + D);
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                const int p = tid + i * kS6Threads;
                const int r = p / (TL::ROWB / 16), c = p % (TL::ROWB / 16);
                r_act[q][i] = __builtin_bit_cast(
                    s6_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                  rs, (uint32_t)(r * act_stride[q] * (int64_t)sizeof(T) + c * 16), 0, 0));
            }
        }
        if (bc_on) {
            const __amdgpu_buffer_rsrc_t rs = s6_rsrc<T>(bc_src, row0 * bc_stride, (rows - 1) * bc_stride + N);
            const int r = bcp / PPR_BC, c = bcp % PPR_BC;
            r_bc = __builtin_bit_cast(s6_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs, (uint32_t)(r * bc_stride * (int64_t)sizeof(T) + c * 16), 0, 0));
        }
        if (doc && tid < TT) {
            const int t = t0 + tid;
            if (t < tend && t > 0) {
                r_doc0 = doc[t];
                r_doc1 = doc[t - 1];
            } else {
                r_doc0 = r_doc1 = 0;
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            if (q == 2 && !has_z) break;
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                const int p = tid + i * kS6Threads;
                reinterpret_cast<s6_u32x4*>(&s_act[q][0][0])[p] = r_act[q][i];
            }
        }
        if (bc_on) {                               // widened to fp32 once here, not in every lane
            constexpr int EPP = 16 / (int)sizeof(T);            // elements per 16-byte piece
            float4* dst = reinterpret_cast<float4*>(&s_bc[bcsel][0][0] + bcp * EPP);
            if (sizeof(T) == 2) {
                dst[0] = make_float4(bf16_lo(r_bc.x), bf16_hi(r_bc.x), bf16_lo(r_bc.y), bf16_hi(r_bc.y));
                dst[EPP / 8] = make_float4(bf16_lo(r_bc.z), bf16_hi(r_bc.z), bf16_lo(r_bc.w), bf16_hi(r_bc.w));
            } else {
                dst[0] = __builtin_bit_cast(float4, r_bc);
            }
        }
        if (tid < 64) {
            const uint64_t m = __ballot(doc != nullptr && tid < TT && r_doc0 != r_doc1);
            if (tid == 0) s_mask = (uint32_t)m;
        }
    };

    float sdt = 0.0f;                              // pre-pass: sum of dt since the last document start
    bool reset = false;                            // pre-pass: a document starts inside the superchunk

    if (tbeg < tend) issue(tbeg);
    for (int t0 = tbeg; t0 < tend; t0 += TT) {
        __syncthreads();                           // the previous tile has been read
        stage();
        __syncthreads();
        if (t0 + TT < tend) issue(t0 + TT);        // in flight during this tile
        const uint32_t mask = __builtin_amdgcn_readfirstlane(s_mask);
        const int nt = min(TT, tend - t0);
        // Per token, the per-channel scalars and the B / C rows of the next
        // token are read and computed in the same block as the current
        // token's state update, so the LDS reads and the dt / gate
        // transcendentals overlap the state arithmetic.
        struct Tok { float dt, dtx, xd, g; float Bt[N], Ct[N]; };
        auto front = [&](int i) {
            Tok o;
            const float raw = s6_ld(&s_act[1][i][tid]);
            const float sp = softplus_hw(raw + bias);
            o.dt = a.dt_softplus ? sp : raw;
            const float xv = s6_ld(&s_act[0][i][tid]);
            o.dtx = o.dt * xv;
            o.xd = Dd * xv;
            o.g = 1.0f;
            if (FULL) {
                const float gz = silu_f(s6_ld(&s_act[NT - 1][i][tid]));
                o.g = has_z ? gz : 1.0f;
                s6_row<N>(&s_bc[1][i][0], o.Ct);
            }
            s6_row<N>(&s_bc[0][i][0], o.Bt);
            return o;
        };
        // y through a range-checked buffer store: lanes past D store out of range
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
            a.y + ((size_t)b * L + t0) * a.y_stride + c0, 0, 0x7fffffff, 0x00020000);
        const uint32_t ylane = on ? (uint32_t)tid * 4u : 0x80000000u;
        Tok cur;
        if (kS6Pipe) cur = front(0);
        // runs of tokens between document starts: the state is cleared once per
        // run, outside the per-token loop
        for (int i = 0; i < nt;) {
            if ((mask >> i) & 1u) {                // uniform: a document starts at t0 + i
#pragma unroll
                for (int n = 0; n < N; ++n) h[n] = 0.0f;
                reset = true;
                sdt = 0.0f;
            }
            const uint32_t rest = (mask >> i) >> 1;
            const int j = rest ? min(nt, i + 1 + (int)__builtin_ctz(rest)) : nt;
            for (; i < j; ++i) {
                Tok nx;
                if (kS6Pipe) nx = front(min(i + 1, nt - 1));
                else cur = front(i);
                if (FULL) {
                    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        h[n] = fmaf(fast_exp2(cur.dt * A2[n]), h[n], cur.dtx * cur.Bt[n]);
                        acc[n & 3] = fmaf(cur.Ct[n], h[n], acc[n & 3]);
                    }
                    const float v = ((acc[0] + acc[1]) + (acc[2] + acc[3]) + cur.xd) * cur.g;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yrs,
                                                          ylane + (uint32_t)(i * a.y_stride) * 4u, 0, 0);
                } else {
#pragma unroll
                    for (int n = 0; n < N; ++n) h[n] = fmaf(fast_exp2(cur.dt * A2[n]), h[n], cur.dtx * cur.Bt[n]);
                    sdt += cur.dt;
                }
                if (kS6Pipe) cur = nx;
            }
        }
    }

    if (!on) return;
    if (FULL) {
        if (a.final_state && k == a.K - 1) {
#pragma unroll
            for (int n = 0; n < N; ++n) a.final_state[sidx * N + n] = h[n];
        }
    } else {
        const size_t u = sidx * (a.K - 1) + k;
#pragma unroll
        for (int n = 0; n < N; ++n) a.hloc[u * N + n] = h[n];
        a.sdt[u] = reset ? -INFINITY : sdt;       // -inf: the incoming state is dropped
    }
}

template <typename T, int N>
hipError_t launch_s6_n(const S6Args& a, hipStream_t stream) {
    const int nblk = (a.D + kS6Threads - 1) / kS6Threads;
    if (a.K > 1) {
        hipLaunchKernelGGL((ssd_s6_kernel<T, N, kS6State>), dim3(a.B * nblk * (a.K - 1)), dim3(kS6Threads), 0,
                           stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((ssd_s6_kernel<T, N, kS6Full>), dim3(a.B * nblk * a.K), dim3(kS6Threads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_s6_t(const S6Args& a, hipStream_t stream) {
    switch (a.N) {
        case 8: return launch_s6_n<T, 8>(a, stream);
        case 16: return launch_s6_n<T, 16>(a, stream);
        case 32: return launch_s6_n<T, 32>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Superchunks: enough workgroups for kS6WgPerCu per CU (256 CUs), at most 32
// and at most one per 64 tokens.
void s6_split(int B, int L, int D, int& K, int& S) {
    const long nblk = (D + kS6Threads - 1) / kS6Threads;
    const long wgs = (long)B * nblk;
    const long target = 256L * kS6WgPerCu;
    long k = (target + wgs - 1) / wgs;
    k = std::max(1L, std::min({k, 32L, (long)(L + 63) / 64}));
    S = (int)((L + k - 1) / k);
    K = (int)((L + S - 1) / S);
}

size_t s6_workspace_bytes(int B, int L, int D, int N) {
    int K, S;
    s6_split(B, L, D, K, S);
    if (K <= 1) return 0;
    const size_t u = (size_t)B * D * (K - 1);
    // hloc [u][N], sdt [u] (padded to 256 bytes), the copy of init_state [B][D][N]
    return u * N * sizeof(float) + (u * sizeof(float) + 255) / 256 * 256 + (size_t)B * D * N * sizeof(float);
}

hipError_t launch_s6(const S6Args& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 0 ? launch_s6_t<float>(a, stream) : launch_s6_t<uint16_t>(a, stream);
}

}  // namespace ssd
