// bwd.hip -- backward (vector-Jacobian product) of the chunked scan and of the
// conv for a zero-state prefill, on gfx950.
//
// The backward of a prefill from a zero state, given dLoss/dy, recomputing the
// forward (mojolearn.Mamba3Block docs, backward(): no gradient for a carried
// state, no final-state cotangent).  Per chunk of 64 tokens and head, with cs
// the cumulative sum of dt*A restarted at each document start, seg(t) the last
// document start in the chunk at or before t (none: -1), Hin the state
// entering the chunk and Gout the adjoint of the state leaving it:
//
//   Lm[t,s]  = exp(cs_t - cs_s) for s <= t in the same segment, else 0
//   M        = (C B^T) o Lm o dt_s            (the chunk's token mixing)
//   in_t     = exp(cs_t) if seg(t) = -1 else 0  (the share of Hin in h_t)
//   el_s     = exp(cs_end - cs_s) if s is in the chunk's last segment, else 0
//   y_t      = (M X + in o (C Hin) + D X)_t * silu(z_t)
//   H_leave  = [seg(end) = -1] exp(cs_end) Hin + sum_s el_s dt_s B_s x_s^T
//
// The backward of these expressions, with dyr = dy o silu(z):
//   dX  = M^T dyr + D dyr + (el o dt) o (B Gout)
//   dB  = dG^T C + (el o dt) o (X Gout^T),  dG = (dyr X^T) o Lm o dt_s
//   dC  = dG B + in o (dyr Hin^T)
//   ddt = colsum((dyr X^T) o G o Lm) + el o u + A * revcumsum_seg(dcs),
//         u_s = B_s^T Gout x_s, dcs from the exponents of Lm, in and el
// Hin and Gout come from two passes over the chunks: the chunk-local states
// S_c = sum_s el_s dt_s B_s x_s^T and the adjoint inputs dS_c = sum_t in_t
// C_t dyr_t^T are computed for every chunk in parallel, then scanned in order
// (Hin) and in reverse order (Gout) per state element.  dB and dC are summed
// over a group's heads inside one workgroup, and the per-head parameter
// gradients (dA, dD, dt_bias) go through per-chunk partial sums reduced in a
// fixed order, so every result is deterministic.
//
// All arithmetic is fp32: the 64x64 products of the chunk kernel and of the
// first pass run on the fp32 MFMA from LDS tiles.
#include <algorithm>
#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kQ = 64;       // chunk
constexpr int kBT = 256;     // threads per workgroup
constexpr int kLD = 68;      // padded row of a 64-wide fp32 tile (16-byte aligned, banks shifted)

__device__ __forceinline__ float ldT(const float* p) { return *p; }
__device__ __forceinline__ float ldT(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float sigmoid_acc(float v) { return 1.0f / (1.0f + expf(-v)); }
__device__ __forceinline__ float silu_acc(float v) { return v * sigmoid_acc(v); }
// d silu / dv = s (1 + v (1 - s)), s = sigmoid(v)
__device__ __forceinline__ float dsilu_acc(float v) {
    const float s = sigmoid_acc(v);
    return s * (1.0f + v * (1.0f - s));
}

// sum over the 16 lanes that share lane / 16
__device__ __forceinline__ float sum16(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}
__device__ __forceinline__ float sum64(float v) {
    v = sum16(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Per-row scalars of one (batch row, head, chunk), computed by one wave: the
// activated dt, the chain factor d dt / d(dt input), the segmented cumulative
// sum of dt*A and the last document start at or before each row.
__device__ __forceinline__ void chunk_rows(const BwdArgs& a, int b, int h, int t0, int Qv, int lane, float& dtv,
                                           float& chain, float& cs, int& seg) {
    const bool valid = lane < Qv;
    const int tg = t0 + lane;
    dtv = 0.0f;
    chain = 1.0f;
    if (valid) {
        const float r = a.dt[((size_t)b * a.L + tg) * a.dt_stride + h];
        if (a.dt_softplus) {
            const float v = r + (a.dt_bias ? a.dt_bias[h] : 0.0f);
            dtv = softplus_f(v);
            chain = sigmoid_acc(v);
        } else {
            dtv = r;
            chain = a.chain_from_dt ? -expm1f(-r) : 1.0f;
        }
    }
    const int f = (valid && tg > 0 && a.doc && a.doc[(size_t)b * a.L + tg] != a.doc[(size_t)b * a.L + tg - 1]) ? 1 : 0;
    cs = dtv * a.A[h];
    seg = f ? lane : -1;
    wave_segscan(cs, f, seg);
}

// A z pointer that is always safe to read: without a gate, gy's rows stand in
// (same row positions in bytes, the values are discarded).
template <typename T>
__device__ __forceinline__ const T* z_or_gy(const BwdArgs& a, int64_t& stride) {
    if (a.z) {
        stride = a.z_stride;
        return static_cast<const T*>(a.z);
    }
    stride = a.gy_stride * (int64_t)(sizeof(float) / sizeof(T));
    return reinterpret_cast<const T*>(a.gy);
}

// Product of a 16-row strip on the fp32 MFMA (16x16x4): acc[c] += A(r0 + ., k)
// B(k, c0 + 16c + .) over k < K (a multiple of 16), c < NC, with the layouts
//   A(i, k) = AT ? A[k * lda + i] : A[i * lda + k]
//   B(k, j) = BT ? Bm[j * ldb + k] : Bm[k * ldb + j]
// (offsets multiples of 4 floats).  Lane (q, i) = (lane / 16, lane % 16) supplies A(r0 + i, 4q..4q+3)
// and B(4q..4q+3, c0 + 16c + i) of each 16-wide K block, and element e of
// acc[c] is the output at row r0 + 4q + e, column c0 + 16c + i.
template <bool AT, bool BT, int NC, int UN = 2>
__device__ __forceinline__ void mfma_strip(f32x4 (&acc)[NC], const float* A, int lda, int r0, const float* Bm,
                                           int ldb, int c0, int K, int q, int li) {
    // UN K blocks per iteration (the chunk kernel picks the most its registers
    // hold without spilling: unrolled fully, a strip hoists every LDS read)
#pragma unroll UN
    for (int kb = 0; kb < K; kb += 16) {
        const int k0 = kb + 4 * q;
        float4 af;
        if (AT) {
            af.x = A[(k0 + 0) * lda + r0 + li];
            af.y = A[(k0 + 1) * lda + r0 + li];
            af.z = A[(k0 + 2) * lda + r0 + li];
            af.w = A[(k0 + 3) * lda + r0 + li];
        } else {
            af = *reinterpret_cast<const float4*>(A + (r0 + li) * lda + k0);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c0 + 16 * c + li;
            float4 bf;
            if (BT) {
                bf = *reinterpret_cast<const float4*>(Bm + col * ldb + k0);
            } else {
                bf.x = Bm[(k0 + 0) * ldb + col];
                bf.y = Bm[(k0 + 1) * ldb + col];
                bf.z = Bm[(k0 + 2) * ldb + col];
                bf.w = Bm[(k0 + 3) * ldb + col];
            }
            acc[c] = mma_f32(acc[c], af, bf);
        }
    }
}

// ---- pass 1: chunk-local states (MODE 0) and adjoint inputs (MODE 1)
template <typename T, int N, int MODE>
__global__ __launch_bounds__(kBT) void ssd_bwd_sums_kernel(BwdArgs a) {
    constexpr int P = 64, LDN = N + 4;
    // W [64][LDN] and V [64][kLD]; after the product the same memory stages the
    // [N][kLD] result so it leaves in whole rows
    static_assert(N * kLD <= kQ * LDN + kQ * kLD, "output staging fits");
    __shared__ __attribute__((aligned(16))) float smem[kQ * LDN + kQ * kLD];
    float* sW = smem;
    float* sV = smem + kQ * LDN;
    __shared__ float s_coef[kQ];
    const int tid = threadIdx.x, nc = a.nc;
    const int c = blockIdx.x % nc;
    const int bh = blockIdx.x / nc;
    const int h = bh % a.H, b = bh / a.H;
    const int g = h / (a.H / a.G);
    constexpr int mode = MODE;
    const int t0 = c * kQ, Qv = min(kQ, a.L - t0);
    const size_t row0 = (size_t)b * a.L + t0;
    // per row: mode 0, the weight el_s dt_s of token s in the chunk's end state;
    // mode 1, the share in_t of the entering state in h_t
    if (tid < 64) {
        float dtv, chain, cs;
        int seg;
        chunk_rows(a, b, h, t0, Qv, tid, dtv, chain, cs, seg);
        const int end = Qv - 1;
        const float cs_end = __shfl(cs, end);
        const int seg_end = __shfl(seg, end);
        float coef = 0.0f;
        if (tid < Qv) coef = mode == 0 ? (seg == seg_end ? expf(cs_end - cs) * dtv : 0.0f) : (seg < 0 ? expf(cs) : 0.0f);
        s_coef[tid] = coef;
        if (mode == 0 && tid == 0) a.dec[((size_t)b * a.H + h) * nc + c] = seg_end < 0 ? expf(cs_end) : 0.0f;
    }
    const T* W = static_cast<const T*>(mode == 0 ? a.Bm : a.Cm);
    const int64_t Ws = mode == 0 ? a.B_stride : a.C_stride;
    float wv[kQ * N / kBT], vv[kQ * P / kBT], zq[kQ * P / kBT];
    int64_t zs;
    const T* zp = z_or_gy<T>(a, zs);
#pragma unroll
    for (int q = 0; q < kQ * N / kBT; ++q) {
        const int i = tid + q * kBT, r = i / N, n = i % N;
        wv[q] = ldT(W + (row0 + min(r, Qv - 1)) * Ws + (size_t)g * N + n);   // coef is 0 past Qv
    }
#pragma unroll
    for (int q = 0; q < kQ * P / kBT; ++q) {
        const int i = tid + q * kBT, p = i % P;
        const size_t rr = row0 + min(i / P, Qv - 1);   // a valid row; rows past Qv carry a zero coef
        vv[q] = mode == 0 ? ldT(static_cast<const T*>(a.x) + rr * a.x_stride + (size_t)h * P + p)
                          : a.gy[rr * a.gy_stride + (size_t)h * P + p];
        zq[q] = mode == 1 ? ldT(zp + rr * zs + (size_t)h * P + p) : 0.0f;
    }
    __syncthreads();                               // s_coef
#pragma unroll
    for (int q = 0; q < kQ * N / kBT; ++q) {
        const int i = tid + q * kBT, r = i / N, n = i % N;
        sW[r * LDN + n] = s_coef[r] * wv[q];
    }
#pragma unroll
    for (int q = 0; q < kQ * P / kBT; ++q) {
        const int i = tid + q * kBT;
        sV[(i / P) * kLD + i % P] = (mode == 1 && a.z) ? vv[q] * silu_acc(zq[q]) : vv[q];
    }
    __syncthreads();
    // [N][64] = W^T V on the fp32 MFMA: the N/16 x 4 output tiles are dealt
    // to the four waves, NC 16-column tiles of one 16-row strip each
    {
        constexpr int NC = N >= 64 ? 4 : N / 16;         // 16-column tiles per strip
        constexpr int RS = N >= 64 ? N / 64 : 1;         // 16-row strips per wave
        const int wave = tid >> 6, lane = tid & 63, q = lane >> 4, li = lane & 15;
        const int c0 = 16 * NC * (wave % (4 / NC));       // the first column (head channel p)
        f32x4 acc[RS][NC] = {};
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const int r0 = 16 * ((wave * NC) / 4 * RS + rs);   // this strip's rows (state index n)
            mfma_strip<true, false, NC>(acc[rs], sW, LDN, r0, sV, kLD, c0, kQ, q, li);
        }
        __syncthreads();                           // every wave is done reading W and V
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const int r0 = 16 * ((wave * NC) / 4 * RS + rs);
#pragma unroll
            for (int cc = 0; cc < NC; ++cc)
#pragma unroll
                for (int e = 0; e < 4; ++e) smem[(r0 + 4 * q + e) * kLD + c0 + 16 * cc + li] = acc[rs][cc][e];
        }
    }
    __syncthreads();
    // the [N][64] result, contiguous in the workspace: 16 bytes per lane, whole rows per instruction
    float* out = (mode == 0 ? a.S : a.dS) + (((size_t)b * a.H + h) * nc + c) * N * P;
#pragma unroll
    for (int u = 0; u < N * P / 4 / kBT; ++u) {
        const int i4 = tid + u * kBT, n = i4 / (P / 4), p = 4 * (i4 % (P / 4));
        *reinterpret_cast<f32x4*>(out + (size_t)n * P + p) = *reinterpret_cast<const f32x4*>(smem + n * kLD + p);
    }
}

// ---- pass 2: states entering each chunk (y = 0, in order) and adjoints of
// the states leaving each chunk (y = 1, in reverse order), per state element.
// The recurrence is serial in the chunks, so the loads run a block of kPD
// chunks ahead of it: the next block's values are in flight while the
// current block's results are stored (one load per chunk in flight would
// leave this pass waiting on memory latency at every chunk).
constexpr int kPD = 8;
template <int N>
__global__ __launch_bounds__(kBT) void ssd_bwd_pass_kernel(BwdArgs a) {
    constexpr int NP = N * 64;
    constexpr int per = NP / kBT;
    const int nc = a.nc;
    const int bh = blockIdx.x / per;
    const int e = (blockIdx.x % per) * kBT + threadIdx.x;
    const float* dec = a.dec + (size_t)bh * nc;
    const bool fwd = blockIdx.y == 0;
    float* X = (fwd ? a.S : a.dS) + (size_t)bh * nc * NP + e;
    // chunk of step i (0 .. nc-1) in this direction
    auto chunk = [&](int i) { return fwd ? i : nc - 1 - i; };
    float acc = 0.0f;
    const int nb = nc / kPD;                      // whole blocks; the rest one chunk at a time
    float v[kPD], d[kPD];
    if (nb > 0) {
#pragma unroll
        for (int j = 0; j < kPD; ++j) {
            v[j] = X[(size_t)chunk(j) * NP];
            d[j] = dec[chunk(j)];
        }
    }
    for (int blk = 0; blk < nb; ++blk) {
        const int i0 = blk * kPD;
        float vn[kPD], dn[kPD];
        const bool more = blk + 1 < nb;           // uniform
        if (more) {
#pragma unroll
            for (int j = 0; j < kPD; ++j) {
                vn[j] = X[(size_t)chunk(i0 + kPD + j) * NP];
                dn[j] = dec[chunk(i0 + kPD + j)];
            }
        }
#pragma unroll
        for (int j = 0; j < kPD; ++j) {
            X[(size_t)chunk(i0 + j) * NP] = acc;
            acc = fmaf(d[j], acc, v[j]);
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < kPD; ++j) {
                v[j] = vn[j];
                d[j] = dn[j];
            }
        }
    }
    for (int i = nb * kPD; i < nc; ++i) {
        const int c = chunk(i);
        const float vv = X[(size_t)c * NP];
        X[(size_t)c * NP] = acc;
        acc = fmaf(dec[c], acc, vv);
    }
}

constexpr int kCT = 512;     // chunk kernel: eight waves

// ---- pass 3: every gradient of one (batch row, group, chunk).  Wave w owns
// rows 16 (w % 4) .. +15 and the column half w / 4 of every [64][.] product:
// a lane holds rows R(e) = 16 (w % 4) + 4q + e (e < 4) at columns
// 32 (w / 4) + 16c + li (c < 2).  Row sums of the two halves meet in LDS and
// are added in a fixed order.
//
// The state dimension is held in LDS in blocks of NB = min(N, 64) columns of B
// and C and NB rows of the states entering / leaving the chunk.  With N = 128
// the two blocks take turns: C B^T sums the two blocks' products, and for each
// head the block still resident from the previous head is used first, so one
// block of B and C is reloaded per head.  Every product that contracts over N
// (C Hin, B Gout) is accumulated over the blocks.  The dB / dC columns of the
// block used first are kept in aB[0] / aC[0], those of the other in aB[1] /
// aC[1]; the two swap when the resident block changes.
template <typename T, int N>
__global__ __launch_bounds__(kCT, 1) void ssd_bwd_chunk_kernel(BwdArgs a) {
    constexpr int P = 64;
    constexpr int NB = N < 64 ? N : 64;
    constexpr int NH = N / NB;
    constexpr int LDN = NB + 4;
    constexpr int NCN = NB / 32 > 0 ? NB / 32 : 1;   // dB / dC tiles per half and block (NB = 16: half 0 only)
    // K blocks per unrolled step of the products: all four where the kernel
    // still fits its 256 registers without spilling (N = 16, 64), else two
    constexpr int UN = (N == 16 || N == 64) ? 4 : 2;
    __shared__ __attribute__((aligned(16))) float sB[kQ * LDN];
    __shared__ __attribute__((aligned(16))) float sC[kQ * LDN];
    __shared__ __attribute__((aligned(16))) float sG[kQ * kLD];
    __shared__ __attribute__((aligned(16))) float sX[kQ * kLD];
    __shared__ __attribute__((aligned(16))) float sDy[kQ * kLD];
    __shared__ __attribute__((aligned(16))) float sM[kQ * kLD];
    __shared__ __attribute__((aligned(16))) float sDG[kQ * kLD];
    __shared__ __attribute__((aligned(16))) float sHin[NB * kLD];
    __shared__ __attribute__((aligned(16))) float sGo[NB * kLD];
    __shared__ float s_dt[kQ], s_cs[kQ], s_chain[kQ];
    __shared__ float s_dcs2[2][kQ], s_u2[2][kQ];   // row sums per column half
    __shared__ int s_seg[kQ];
    __shared__ float s_red[2][4][kQ];
    __shared__ float s_scal[2][8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, li = lane & 15;
    const int r0 = 16 * (wave & 3);                // this wave's rows
    const int half = wave >> 2, c0 = 32 * half;    // and column half
    const int nc = a.nc;
    const int c = blockIdx.x % nc;
    const int bg = blockIdx.x / nc;
    const int g = bg % a.G, b = bg / a.G;
    const int hpg = a.H / a.G;
    const int t0 = c * kQ, Qv = min(kQ, a.L - t0);
    const size_t row0 = (size_t)b * a.L + t0;
    // the [64][NB] products (dB, dC) split their NB columns the same way: NB/2
    // per half (NB = 16: one tile, half 0 only)
    const bool nact = NB >= 32 || half == 0;
    const int c0N = NB >= 32 ? half * (NB / 2) : 0;
    auto R = [&](int e) { return r0 + 4 * q + e; };

    // into LDS: block k of the group's B and C rows (fp32, zero past the valid
    // rows) if bc, and block k of the states entering and leaving the chunk of
    // the head at bhc (rows n = k NB .. +NB of [N][P]) if st; every load is
    // issued before the first LDS write
    constexpr int NU = kQ * NB / kCT;
    constexpr int NS4 = (NB * P / 4 + kCT - 1) / kCT;
    auto stage = [&](size_t bhc, int k, bool bc, bool st) __attribute__((always_inline)) {
        // the thread index, opaque to the compiler: the addresses below are
        // rebuilt at every call instead of being hoisted out of the head loop
        // and held in registers across it (which made the N = 128 kernel spill)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        float bv[NU], cv[NU];
        f32x4 hv[NS4], ov[NS4];
        if (bc) {
            // the chunk's rows from a uniform base: offsets within 64 rows fit in 32 bits
            const T* Bb = static_cast<const T*>(a.Bm) + row0 * a.B_stride + (size_t)g * N + k * NB;
            const T* Cb = static_cast<const T*>(a.Cm) + row0 * a.C_stride + (size_t)g * N + k * NB;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int i = tid + u * kCT, r = min(i / NB, Qv - 1), n = i % NB;
                bv[u] = ldT(Bb + (uint32_t)(r * (uint32_t)a.B_stride + n));
                cv[u] = ldT(Cb + (uint32_t)(r * (uint32_t)a.C_stride + n));
            }
        }
        if (st) {
#pragma unroll
            for (int u = 0; u < NS4; ++u) {
                const int i4 = min(tid + u * kCT, NB * P / 4 - 1);
                const uint32_t o = (uint32_t)(k * NB * P + 4 * i4);
                hv[u] = *reinterpret_cast<const f32x4*>(a.S + bhc * N * P + o);
                ov[u] = *reinterpret_cast<const f32x4*>(a.dS + bhc * N * P + o);
            }
        }
        if (bc) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int i = tid + u * kCT, r = i / NB, n = i % NB;   // rows past Qv: zero
                sB[r * LDN + n] = r < Qv ? bv[u] : 0.0f;
                sC[r * LDN + n] = r < Qv ? cv[u] : 0.0f;
            }
        }
        if (st) {
#pragma unroll
            for (int u = 0; u < NS4; ++u) {
                const int i4 = tid + u * kCT;
                if (i4 < NB * P / 4) {
                    const int n = 4 * i4 / P, p = 4 * i4 % P;
                    *reinterpret_cast<f32x4*>(sHin + n * kLD + p) = hv[u];
                    *reinterpret_cast<f32x4*>(sGo + n * kLD + p) = ov[u];
                }
            }
        }
    };
    // <Gout, Hin> over the resident block: this thread's share
    auto state_dot = [&]() __attribute__((always_inline)) {
        float v = 0.0f;
        for (int i = tid; i < NB * P; i += kCT) v = fmaf(sHin[(i / P) * kLD + i % P], sGo[(i / P) * kLD + i % P], v);
        return v;
    };

    // G = C B^T, summed over the blocks
    {
        f32x4 acc[2] = {};
#pragma unroll
        for (int k = 0; k < NH; ++k) {
            if (k) __syncthreads();                // every wave is done with the previous block
            stage(0, k, true, false);
            __syncthreads();
            mfma_strip<false, true, 2, UN>(acc, sC, LDN, r0, sB, LDN, c0, NB, q, li);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[R(e) * kLD + c0 + 16 * cc + li] = acc[cc][e];
    }
    f32x4 aB[NH][NCN] = {}, aC[NH][NCN] = {};     // dB, dC of the group, summed over its heads
    int cur = NH - 1;                              // the block of B and C in LDS (aB[0], aC[0])

    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const float Ah = a.A[h], Dh = a.D ? a.D[h] : 0.0f;
        const size_t bhc = ((size_t)b * a.H + h) * nc + c;
        if (wave == 0) {
            float dtv, chain, cs;
            int seg;
            int ln = lane;                         // opaque, as in stage(): the row pointers are per head
            asm volatile("" : "+v"(ln));
            chunk_rows(a, b, h, t0, Qv, ln, dtv, chain, cs, seg);
            s_dt[lane] = dtv;
            s_cs[lane] = cs;
            s_seg[lane] = seg;
            s_chain[lane] = chain;
        }
        // x, dyr = dy silu(z) and qd = dy silu'(z) at this lane's elements, so
        // dz = qd o y needs no reload; the resident block of the states
        float qd[2][4];
        {
            int64_t zs;
            const T* zp = z_or_gy<T>(a, zs) + row0 * zs;
            const T* xp = static_cast<const T*>(a.x) + row0 * a.x_stride;
            const float* gp = a.gy + row0 * a.gy_stride;
            float xv[2][4], gv[2][4], zv[2][4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t rr = min(R(e), Qv - 1);   // a valid row; zeroed below past Qv
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const uint32_t col = h * P + c0 + 16 * cc + li;
                    xv[cc][e] = ldT(xp + (rr * (uint32_t)a.x_stride + col));
                    gv[cc][e] = gp[rr * (uint32_t)a.gy_stride + col];
                    zv[cc][e] = ldT(zp + (rr * (uint32_t)zs + col));
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = R(e) < Qv;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const float zz = zv[cc][e], gg = ok ? gv[cc][e] : 0.0f;
                    const int o = R(e) * kLD + c0 + 16 * cc + li;
                    sX[o] = ok ? xv[cc][e] : 0.0f;
                    sDy[o] = a.z ? gg * silu_acc(zz) : gg;
                    qd[cc][e] = a.z ? gg * dsilu_acc(zz) : 0.0f;
                }
            }
            stage(bhc, cur, false, true);
        }
        __syncthreads();

        float hg = state_dot();                    // <Gout, Hin> partial
        const int end = Qv - 1;
        const float cs_end = s_cs[end];
        const int seg_end = s_seg[end];
        float in_r[4], we_r[4];                    // in_t, and el_s dt_s, of this lane's rows
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = R(e), sg = s_seg[t];
            in_r[e] = (t < Qv && sg < 0) ? expf(s_cs[t]) : 0.0f;
            we_r[e] = (t < Qv && sg == seg_end) ? expf(cs_end - s_cs[t]) * s_dt[t] : 0.0f;
        }
        auto lmask = [&](int e, int s) {
            const int t = R(e);
            return (s <= t && s_seg[s] == s_seg[t]) ? expf(s_cs[t] - s_cs[s]) : 0.0f;
        };
        // M = G o Lm o dt_s
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int t = R(e), s = c0 + 16 * cc + li;
                sM[t * kLD + s] = sG[t * kLD + s] * lmask(e, s) * s_dt[s];
            }
        __syncthreads();

        float rowD[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // this half's share of dcs per row
        // dM = dyr X^T -> dG, the Lm share of dcs, the direct share of ddt
        {
            f32x4 dm[2] = {};
            mfma_strip<false, true, 2, UN>(dm, sDy, kLD, r0, sX, kLD, c0, P, q, li);
            float colT[2] = {0.0f, 0.0f}, colD[2] = {0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = R(e);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int s = c0 + 16 * cc + li;
                    const float d = dm[cc][e];
                    const float tt = d * sM[t * kLD + s];
                    const float lm = lmask(e, s);
                    rowD[e] += tt;
                    colT[cc] += tt;
                    colD[cc] = fmaf(d, sG[t * kLD + s] * lm, colD[cc]);
                    sDG[t * kLD + s] = d * lm * s_dt[s];
                }
            }
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                float v = colT[cc], w = colD[cc];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                w += __shfl_xor(w, 16);
                w += __shfl_xor(w, 32);
                if (q == 0) {
                    s_red[0][wave & 3][c0 + 16 * cc + li] = v;
                    s_red[1][wave & 3][c0 + 16 * cc + li] = w;
                }
            }
        }
        __syncthreads();                           // dG

        // the products over the state dimension, block by block:
        //   y_off = C Hin, B Gout (accumulated);  dB += dG^T C + (el o dt) o (X Gout^T),
        //   dC += dG B + in o (dyr Hin^T) (the block's columns)
        f32x4 y2[2] = {}, bgo[2] = {};
        auto block = [&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;   // 0: the block used first
            mfma_strip<false, false, 2, UN>(y2, sC, LDN, r0, sHin, kLD, c0, NB, q, li);
            mfma_strip<false, false, 2, UN>(bgo, sB, LDN, r0, sGo, kLD, c0, NB, q, li);
            if (nact) {
                mfma_strip<true, false, NCN, UN>(aB[k], sDG, kLD, r0, sC, LDN, c0N, kQ, q, li);
                mfma_strip<false, false, NCN, UN>(aC[k], sDG, kLD, r0, sB, LDN, c0N, kQ, q, li);
                f32x4 xg[NCN] = {}, dh[NCN] = {};
                mfma_strip<false, true, NCN, UN>(xg, sX, kLD, r0, sGo, kLD, c0N, P, q, li);
                mfma_strip<false, true, NCN, UN>(dh, sDy, kLD, r0, sHin, kLD, c0N, P, q, li);
#pragma unroll
                for (int cc = 0; cc < NCN; ++cc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        aB[k][cc][e] = fmaf(we_r[e], xg[cc][e], aB[k][cc][e]);
                        aC[k][cc][e] = fmaf(in_r[e], dh[cc][e], aC[k][cc][e]);
                    }
            }
        };
        block(std::integral_constant<int, 0>{});
        if constexpr (NH == 2) {
            const int nxt = 1 - cur;
            __syncthreads();                       // every wave is done with the resident block
            stage(bhc, nxt, true, true);
            __syncthreads();
            hg += state_dot();
            block(std::integral_constant<int, 1>{});
            cur = nxt;                             // now resident: used first by the next head
#pragma unroll
            for (int cc = 0; cc < NCN; ++cc) {
                const f32x4 tb = aB[0][cc], tc = aC[0][cc];
                aB[0][cc] = aB[1][cc];
                aC[0][cc] = aC[1][cc];
                aB[1][cc] = tb;
                aC[1][cc] = tc;
            }
        }

        // y (before the gate) = M X + in o (C Hin) + D X; dz; the in_t share of dcs; dD;
        // dX = M^T dyr + D dyr + (el o dt) o (B Gout); u_s = (B Gout)_s . x_s
        {
            f32x4 y1[2] = {}, d1[2] = {};
            mfma_strip<false, false, 2, UN>(y1, sM, kLD, r0, sX, kLD, c0, kQ, q, li);
            mfma_strip<true, false, 2, UN>(d1, sM, kLD, r0, sDy, kLD, c0, kQ, q, li);
            float pD = 0.0f;
            float ru[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = R(e);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int p = c0 + 16 * cc + li;
                    const float xv = sX[t * kLD + p], dy = sDy[t * kLD + p];
                    rowD[e] = fmaf(in_r[e] * y2[cc][e], dy, rowD[e]);
                    pD = fmaf(dy, xv, pD);
                    ru[e] = fmaf(bgo[cc][e], xv, ru[e]);
                    if (t < Qv) {
                        const uint32_t col = h * P + p;
                        if (a.dz)
                            a.dz[row0 * a.dz_stride + (t * (uint32_t)a.dz_stride + col)] =
                                qd[cc][e] * (y1[cc][e] + in_r[e] * y2[cc][e] + Dh * xv);
                        a.dx[row0 * a.dx_stride + (t * (uint32_t)a.dx_stride + col)] =
                            d1[cc][e] + Dh * dy + we_r[e] * bgo[cc][e];
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = sum16(rowD[e]);
                const float u = sum16(ru[e]);
                if (li == 0) {
                    s_dcs2[half][R(e)] = v;
                    s_u2[half][R(e)] = u;
                }
            }
            pD = sum64(pD);
            hg = sum64(hg);
            if (lane == 0) {
                s_scal[0][wave] = pD;
                s_scal[1][wave] = hg;
            }
        }
        __syncthreads();

        // per row: the el share of dcs and ddt, the reverse segmented cumsum of
        // dcs into ddt and dA, the chain to the dt input, the partial sums
        if (wave == 0) {
            const int t = lane;
            const bool valid = t < Qv;
            const float el = (valid && s_seg[t] == seg_end) ? expf(cs_end - s_cs[t]) : 0.0f;
            const float dtv = s_dt[t], u = s_u2[0][t] + s_u2[1][t];
            const float wu = el * dtv * u;
            const float colsumT = (s_red[0][0][t] + s_red[0][1][t]) + (s_red[0][2][t] + s_red[0][3][t]);
            float dcs = (s_dcs2[0][t] + s_dcs2[1][t]) - colsumT - wu;
            const float sum_wu = sum64(wu);
            const float hgt = ((s_scal[1][0] + s_scal[1][1]) + (s_scal[1][2] + s_scal[1][3])) +
                              ((s_scal[1][4] + s_scal[1][5]) + (s_scal[1][6] + s_scal[1][7]));
            if (t == end) dcs += sum_wu + (seg_end < 0 ? expf(cs_end) : 0.0f) * hgt;
            float ddt = (s_red[1][0][t] + s_red[1][1][t]) + (s_red[1][2][t] + s_red[1][3][t]) + el * u;
            // segments in reverse order start where the original row ends one
            const int fend = (t == kQ - 1 || s_seg[t + 1 < kQ ? t + 1 : t] == t + 1) ? 1 : 0;
            float vr = __shfl(dcs, 63 - lane);
            const int fr = __shfl(fend, 63 - lane);
            int sr = fr ? lane : -1;
            wave_segscan(vr, fr, sr);
            const float rc = __shfl(vr, 63 - lane);
            ddt = fmaf(Ah, rc, ddt);
            const float pA = sum64(valid ? dtv * rc : 0.0f);
            const float dout = ddt * s_chain[t];
            const float pBias = sum64(valid ? dout : 0.0f);
            if (valid) a.ddt[(row0 + t) * a.ddt_stride + h] = dout;
            if (lane == 0) {
                const size_t bc = (size_t)b * nc + c;
                const size_t nbc = (size_t)a.B * nc;
                a.part[(0 * nbc + bc) * a.H + h] = pA;
                a.part[(1 * nbc + bc) * a.H + h] = ((s_scal[0][0] + s_scal[0][1]) + (s_scal[0][2] + s_scal[0][3])) +
                                                    ((s_scal[0][4] + s_scal[0][5]) + (s_scal[0][6] + s_scal[0][7]));
                a.part[(2 * nbc + bc) * a.H + h] = pBias;
            }
        }
        __syncthreads();
    }
    if (nact) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = R(e);
            if (r < Qv) {
#pragma unroll
                for (int k = 0; k < NH; ++k)
#pragma unroll
                    for (int cc = 0; cc < NCN; ++cc) {
                        const int blk = k == 0 ? cur : NH - 1 - cur;
                        const size_t col = (size_t)g * N + blk * NB + c0N + 16 * cc + li;
                        a.dB[row0 * a.dB_stride + (r * (uint32_t)a.dB_stride + (uint32_t)col)] = aB[k][cc][e];
                        a.dC[row0 * a.dC_stride + (r * (uint32_t)a.dC_stride + (uint32_t)col)] = aC[k][cc][e];
                    }
            }
        }
    }
}

// Fixed-order sums of the per-chunk partials part[q][i][k] (q < 3, i < rows,
// k < per) into o_q[k]: 16 columns per workgroup, each summed by 16 threads
// over interleaved rows, then the 16 partials added in order.
__global__ __launch_bounds__(kBT) void ssd_bwd_reduce_kernel(const float* part, int rows, int per, float* o0,
                                                             float* o1, float* o2) {
    __shared__ float s_p[16][16];
    const int col = threadIdx.x & 15, sl = threadIdx.x >> 4;
    const int j = blockIdx.x * 16 + col;
    const bool on = j < 3 * per;
    const int q = on ? j / per : 0, k = on ? j % per : 0;
    float s = 0.0f;
    if (on)
        for (int i = sl; i < rows; i += 16) s += part[((size_t)q * rows + i) * per + k];
    s_p[sl][col] = s;
    __syncthreads();
    if (sl == 0 && on) {
        float t = 0.0f;
        for (int u = 0; u < 16; ++u) t += s_p[u][col];
        float* o = q == 0 ? o0 : (q == 1 ? o1 : o2);
        if (o) o[k] = t;
    }
}

__global__ __launch_bounds__(kBT) void ssd_zero_kernel(float* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * kBT + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ---- conv backward: one channel per thread, 64 tokens per workgroup
constexpr int kCB = 256;     // channels per workgroup

// d silu / dv with the hardware exp2 and reciprocal (a few ulp)
__device__ __forceinline__ float dsilu_fast(float v) {
    const float s = fast_rcp(1.0f + fast_exp2(-v * kLog2e));
    return s * (1.0f + v * (1.0f - s));
}

template <typename T>
__global__ __launch_bounds__(kCB) void ssd_conv_bwd_kernel(ConvBwdArgs a) {
    constexpr int K = 4, TC = 64, U = 8;
    __shared__ unsigned long long s_mask[2];       // document starts at rows t0 - 3 + i, i < 128
    const int C = a.C, L = a.L, tid = threadIdx.x;
    const int nblk = (C + kCB - 1) / kCB;
    const int blk = blockIdx.x % nblk;
    const int tc = (blockIdx.x / nblk) % a.ntc;
    const int b = blockIdx.x / (nblk * a.ntc);
    const int c = blk * kCB + tid;
    const bool on = c < C;
    const int cc = min(c, C - 1);
    const int t0 = tc * TC, t1 = min(t0 + TC, L);
    const int32_t* docb = a.doc ? a.doc + (size_t)b * L : nullptr;
    if (tid < 64) {
        auto start = [&](int t) { return docb && t > 0 && t < L && docb[t] != docb[t - 1]; };
        const unsigned long long lo = __ballot(start(t0 - (K - 1) + tid));
        const unsigned long long hi = __ballot(start(t0 - (K - 1) + 64 + tid));
        if (tid == 0) {
            s_mask[0] = lo;
            s_mask[1] = hi;
        }
    }
    __syncthreads();
    // (readfirstlane returns a signed int: widen through uint32_t)
    auto uniform64 = [](unsigned long long v) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return ((uint64_t)hi << 32) | lo;
    };
    const uint64_t mlo = uniform64(s_mask[0]);
    const uint64_t mhi = uniform64(s_mask[1]);
    auto start_at = [&](int t) {                   // uniform: a document starts at row t
        const int i = t - t0 + K - 1;
        return ((i < 64 ? mlo >> i : mhi >> (i - 64)) & 1u) != 0;
    };
    float w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = a.w[(size_t)cc * K + k];
    const float bias = a.bias ? a.bias[cc] : 0.0f;
    const T* rawb = static_cast<const T*>(a.raw) + (size_t)b * L * a.raw_stride + cc;
    const float* doutb = a.dout + (size_t)b * L * a.dout_stride + cc;
    float* drawb = a.draw + (size_t)b * L * a.draw_stride + c;
    // raw rows t-3 .. t (0 before row 0) and d(pre-activation) of rows t-3 .. t
    float win[K], dp[K] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        const int t = t0 - (K - 1) + k;
        const float v = ldT(rawb + (size_t)max(t, 0) * a.raw_stride);
        win[k + 1] = t < 0 ? 0.0f : v;
    }
    float gw[K] = {0.0f, 0.0f, 0.0f, 0.0f}, gb = 0.0f;
    // Rows t0 .. t1 + 2: dpre[t] for t < L (the three rows past the tile feed
    // the tile's last draw rows), and draw[t - 3] as soon as dpre[t] is known.
    // Two register sets of loads are used in turn, one block ahead.
    const int tEnd = t1 + K - 1;
    float ra[U], ga[U], rb[U], gb2[U];
    auto load_block = [&](int tb, float* r, float* gg) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tl = min(tb + u, L - 1);     // rows past the end load a valid row, unused
            r[u] = ldT(rawb + (size_t)tl * a.raw_stride);
            gg[u] = doutb[(size_t)tl * a.dout_stride];
        }
    };
    auto compute_block = [&](int tb, const float* rv, const float* gv) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tb + u;
            if (t >= tEnd) break;
#pragma unroll
            for (int k = 0; k < K - 1; ++k) {
                win[k] = win[k + 1];
                dp[k] = dp[k + 1];
            }
            win[K - 1] = rv[u];
            // tap k reads row t - 3 + k: valid if it is a row (>= 0) and no
            // document starts in (t - 3 + k, t]
            bool ok[K];
            ok[K - 1] = true;
            bool run = true;
#pragma unroll
            for (int k = K - 2; k >= 0; --k) {
                run = run && !start_at(t - (K - 1) + k + 1);
                ok[k] = run && t - (K - 1) + k >= 0;
            }
            float pre = bias;
#pragma unroll
            for (int k = 0; k < K; ++k) pre = fmaf(w[k], ok[k] ? win[k] : 0.0f, pre);
            const float gp = t < L ? (a.act == 0 ? gv[u] * dsilu_fast(pre) : gv[u]) : 0.0f;
            dp[K - 1] = gp;
            if (t < t1) {
                gb += gp;
#pragma unroll
                for (int k = 0; k < K; ++k) gw[k] = fmaf(gp, ok[k] ? win[k] : 0.0f, gw[k]);
            }
            // draw[s], s = t - 3: sum over the taps k that read row s, of the
            // tokens s + 3 - k (dp[3 - k]) with no document start in (s, s + 3 - k]
            const int s = t - (K - 1);
            if (s >= t0) {
                float acc = w[K - 1] * dp[0];
                bool r2 = true;
#pragma unroll
                for (int k = K - 2; k >= 0; --k) {
                    r2 = r2 && !start_at(s + (K - 1) - k);
                    acc = fmaf(w[k], r2 ? dp[K - 1 - k] : 0.0f, acc);
                }
                if (on) drawb[(size_t)s * a.draw_stride] = acc;
            }
        }
    };
    load_block(t0, ra, ga);
    for (int tb = t0; tb < tEnd; tb += 2 * U) {
        load_block(tb + U, rb, gb2);
        compute_block(tb, ra, ga);
        load_block(tb + 2 * U, ra, ga);
        compute_block(tb + U, rb, gb2);
    }
    if (on) {
        float* pp = a.part + (((size_t)b * a.ntc + tc) * C + c) * (K + 1);
#pragma unroll
        for (int k = 0; k < K; ++k) pp[k] = gw[k];
        pp[K] = gb;
    }
}

// dw[c][k] and dbias[c] from the per-chunk partials [rows][C][5], reduced as
// in ssd_bwd_reduce_kernel
__global__ __launch_bounds__(kBT) void ssd_conv_bwd_reduce_kernel(const float* part, int rows, int C, float* dw,
                                                                  float* dbias) {
    __shared__ float s_p[16][16];
    const int col = threadIdx.x & 15, sl = threadIdx.x >> 4;
    const int j = blockIdx.x * 16 + col;
    const bool on = j < C * 5;
    float s = 0.0f;
    if (on)
        for (int i = sl; i < rows; i += 16) s += part[(size_t)i * C * 5 + j];
    s_p[sl][col] = s;
    __syncthreads();
    if (sl == 0 && on) {
        float t = 0.0f;
        for (int u = 0; u < 16; ++u) t += s_p[u][col];
        const int c = j / 5, k = j % 5;
        if (k < 4) dw[(size_t)c * 4 + k] = t;
        else if (dbias) dbias[c] = t;
    }
}

template <typename T, int N>
hipError_t launch_bwd_n(const BwdArgs& a, hipStream_t stream) {
    const int bhc = a.B * a.H * a.nc;
    hipLaunchKernelGGL((ssd_bwd_sums_kernel<T, N, 0>), dim3(bhc), dim3(kBT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_bwd_sums_kernel<T, N, 1>), dim3(bhc), dim3(kBT), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_bwd_pass_kernel<N>), dim3(a.B * a.H * (N * 64 / kBT), 2), dim3(kBT), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_bwd_chunk_kernel<T, N>), dim3(a.B * a.G * a.nc), dim3(kCT), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((3 * a.H + 15) / 16), dim3(kBT), 0, stream, a.part,
                       a.B * a.nc, a.H, a.dA, a.dD, a.ddt_bias);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_bwd_n<T, 16>(a, stream);
        case 32: return launch_bwd_n<T, 32>(a, stream);
        case 64: return launch_bwd_n<T, 64>(a, stream);
        case 128: return launch_bwd_n<T, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t scan_bwd_workspace_bytes(int B, int L, int H, int P, int N) {
    const size_t nc = (size_t)(L + kQ - 1) / kQ;
    const size_t st = (size_t)B * H * nc * N * P * sizeof(float);
    auto r256 = [](size_t n) { return (n + 255) / 256 * 256; };
    return 2 * r256(st) + r256((size_t)B * H * nc * sizeof(float)) + r256(3 * (size_t)B * nc * H * sizeof(float));
}

hipError_t launch_scan_bwd(const BwdArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.L == 0) return hipSuccess;
    return a.dtype == 0 ? launch_bwd_t<float>(a, stream) : launch_bwd_t<uint16_t>(a, stream);
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream) {
    if (!p || n == 0) return hipSuccess;
    hipLaunchKernelGGL(ssd_zero_kernel, dim3((unsigned)((n + kBT - 1) / kBT)), dim3(kBT), 0, stream, p, n);
    return hipGetLastError();
}

size_t conv_bwd_workspace_bytes(int B, int L, int C) {
    const size_t ntc = (size_t)(L + 63) / 64;
    return (size_t)B * ntc * C * 5 * sizeof(float);
}

hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.L == 0) return hipSuccess;
    const int nblk = (a.C + kCB - 1) / kCB;
    if (a.dtype == 0)
        hipLaunchKernelGGL((ssd_conv_bwd_kernel<float>), dim3(a.B * a.ntc * nblk), dim3(kCB), 0, stream, a);
    else
        hipLaunchKernelGGL((ssd_conv_bwd_kernel<uint16_t>), dim3(a.B * a.ntc * nblk), dim3(kCB), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ssd_conv_bwd_reduce_kernel, dim3((a.C * 5 + 15) / 16), dim3(kBT), 0, stream, a.part,
                       a.B * a.ntc, a.C, a.dw, a.dbias);
    return hipGetLastError();
}

}  // namespace ssd
