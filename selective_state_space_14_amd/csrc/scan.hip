// scan.hip -- ssd_chunk_scan_fwd: the Mamba-2 SSD selective scan on gfx950.
//
// Recurrence (per batch row b, head h in group g):
//     h_t = exp(dt_t A_h) h_{t-1} + dt_t B_t x_t^T,   y_t = (C_t . h_t + D_h x_t) silu(z_t)
// evaluated in chunks of Q = 64 tokens with the dual (quadratic) form inside
// a chunk and the state passed between chunks (chunk size 64: the
// mojolearn.Mamba3Block description; the layer itself: the Codestral-Mamba
// port header and the Mini-K3-1H card).
//
// Work decomposition: one workgroup = one (b, h) = 4 waves; wave w owns the
// 16 head channels p in [16w, 16w+16) for the whole sequence and keeps their
// slice of the fp32 state H (N x 16) in registers.  Chunks are walked strictly
// in order, so the state never leaves the chip and a prefill split at a
// multiple of 64 tokens reproduces one call bit for bit.  Per chunk c with
// tokens t, s in [0, 64) (cs = log2-domain cumulative sum of dt A, restarted
// at every document start inside the chunk):
//   G^T[s,t]  = B_s . C_t                       (MFMA, K = N; 10 lower tiles,
//                                                 split over the 4 waves)
//   M^T[s,t]  = G^T[s,t] 2^(cs_t - cs_s) dt_s    for seg(t) <= s <= t, else 0
//   Ydiag^T   = X^T M^T                          (MFMA, K = s)
//   Yoff^T    = H_prev^T C^T                     (MFMA, K = N; H split into
//                                                 bf16 hi + lo parts)
//   S         = B^T (w o X),  w_s = 2^(cs_end - cs_s) dt_s on the last segment
//   y_t       = Ydiag + [t in a carried segment] 2^(cs_t) Yoff + D x_t, gated
//   H         = chunk holds a boundary ? S : 2^(cs_end) H_prev + S
// Every document mask is a select, never a multiply, so tokens of a later
// document are bit-for-bit independent of (finite) earlier-document inputs.
// The pairwise decay is built from the difference cs_t - cs_s (the two sums
// alone can reach hundreds in magnitude within a chunk).
//
// All contractions are 16x16 MFMA tiles whose accumulator layout doubles as
// the next contraction's operand layout (see ssd_device.hpp), so G^T feeds
// the Y contraction and H feeds the C.H contraction without any shuffle.
// LDS holds B (row-major and transposed), C, X^T, (w o X)^T, the M^T tiles
// and the chunk's cs/dt/segment arrays; the next chunk's global loads are
// issued right after staging, so they fly during the contractions.
#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int Q = 64;            // chunk length
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPad = 4;          // row padding (elements) of every LDS matrix
constexpr int kXS = Q + kPad;    // row stride of the s-contiguous matrices
constexpr int kNumMTiles = 10;   // 16x16 tiles (si <= ti) of the 64x64 lower triangle

template <typename T> struct Tr;
template <> struct Tr<uint16_t> {          // bf16 storage
    using E = uint16_t;
    using Frag = FragBF;
    using Raw4 = uint2;                    // 4 consecutive elements
    static constexpr int VE = 8;           // elements per 16 bytes
    __device__ static Frag ld(const E* p) { const uint2 v = *reinterpret_cast<const uint2*>(p); return {v.x, v.y}; }
    __device__ static Frag zero() { return {0u, 0u}; }
    __device__ static Frag from_acc(f32x4 v) { return frag_from_f32(v); }
    __device__ static f32x4 mma2(f32x4 acc, Frag a0, Frag a1, Frag b0, Frag b1) { return mma_bf16(acc, a0, a1, b0, b1); }
    __device__ static float el(Raw4 v, int r) {
        const uint32_t w = r < 2 ? v.x : v.y;
        return (r & 1) ? bf16_hi(w) : bf16_lo(w);
    }
    __device__ static E from_f(float v) { return (E)f32_to_bf16_bits(v); }
    __device__ static E raw_el(Raw4 v, int r) {
        const uint32_t w = r < 2 ? v.x : v.y;
        return (E)((r & 1) ? (w >> 16) : (w & 0xffffu));
    }
    __device__ static Raw4 zero4() { return make_uint2(0u, 0u); }
    // two elements of consecutive rows, packed for one LDS store
    __device__ static uint32_t pair(uint4 lo_row, uint4 hi_row, int e) {
        const uint32_t a = (&lo_row.x)[e >> 1], b = (&hi_row.x)[e >> 1];
        return (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    using Pair = uint32_t;
};
template <> struct Tr<float> {             // fp32 storage
    using E = float;
    using Frag = float4;
    using Raw4 = float4;
    static constexpr int VE = 4;
    __device__ static Frag ld(const E* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static Frag zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ static Frag from_acc(f32x4 v) { return make_float4(v[0], v[1], v[2], v[3]); }
    __device__ static f32x4 mma2(f32x4 acc, Frag a0, Frag a1, Frag b0, Frag b1) {
        acc = mma_f32(acc, a0, b0);
        return mma_f32(acc, a1, b1);
    }
    __device__ static float el(Raw4 v, int r) { return (&v.x)[r]; }
    __device__ static E from_f(float v) { return v; }
    __device__ static E raw_el(Raw4 v, int r) { return (&v.x)[r]; }
    __device__ static Raw4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ static float2 pair(uint4 lo_row, uint4 hi_row, int e) {
        return make_float2(__uint_as_float((&lo_row.x)[e]), __uint_as_float((&hi_row.x)[e]));
    }
    using Pair = float2;
};

// Tiles of the lower triangle, dealt round-robin to the waves: tile k -> (si, ti).
// Order: diagonal tiles first, then (0,1) (0,2) (0,3) (1,2) (1,3) (2,3); the
// table lives in two immediates (4 bits per tile) so no memory is touched.
__device__ __forceinline__ void mtile(int k, int& si, int& ti) {
    constexpr unsigned long long kS = 0x2110003210ull;   // si of tile k in nibble k
    constexpr unsigned long long kT = 0x3323213210ull;   // ti of tile k in nibble k
    si = (int)((kS >> (4 * k)) & 0xF);
    ti = (int)((kT >> (4 * k)) & 0xF);
}
__device__ __forceinline__ int mtile_index(int si, int ti) {
    return si == ti ? si : (si == 0 ? 3 + ti : (si == 1 ? 5 + ti : 9));
}

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so that a
// contiguous range of (b, h) -- heads of the same group, which share B and C
// -- runs on one XCD and shares its L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    const int q = n / 8, r = n % 8;
    const int xcd = i % 8, slot = i / 8;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

template <typename T, int N>
struct Lds {
    using E = typename Tr<T>::E;
    static constexpr int NS = N + kPad;                 // row stride of B and C
    static constexpr size_t oB = 0;                     // B   [Q][NS]
    static constexpr size_t oC = oB + (size_t)Q * NS;   // C   [Q][NS]
    static constexpr size_t oBt = oC + (size_t)Q * NS;  // B^T [N][kXS]
    static constexpr size_t oXt = oBt + (size_t)N * kXS;        // X^T   [64 p][kXS]
    static constexpr size_t oXwt = oXt + (size_t)64 * kXS;      // (wX)^T [64 p][kXS]
    static constexpr size_t oM = oXwt + (size_t)64 * kXS;       // M^T tiles [10][64 lanes][4]
    static constexpr size_t nE = oM + (size_t)kNumMTiles * 256;
    // per-token scalars: cs, dt, segment start, Yoff scale, chunk-state weight
    static constexpr size_t bytes = nE * sizeof(E) + 5 * Q * sizeof(float);
};

template <typename T, int N>
struct ChunkRegs {
    using R = Tr<T>;
    static constexpr int CPR = N * (int)sizeof(typename R::E) / 16;   // 16-byte chunks per B/C row
    static constexpr int NITEMS = 32 * CPR;                            // (row pair, chunk) items
    static constexpr int NIT = (NITEMS + kThreads - 1) / kThreads;
    uint4 b[NIT][2], c[NIT][2];
    typename R::Raw4 x[4], z[4];
    float dt;
    int d0, d1;       // document id of the token and of the one before it
};

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(ScanArgs a) {
    using R = Tr<T>;
    using E = typename R::E;
    using Frag = typename R::Frag;
    using Raw4 = typename R::Raw4;
    using LD = Lds<T, N>;
    using CR = ChunkRegs<T, N>;
    constexpr int NT = N / 16;            // n tiles
    constexpr int NS = LD::NS;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    E* sm = reinterpret_cast<E*>(smem_raw);
    E* sB = sm + LD::oB;
    E* sC = sm + LD::oC;
    E* sBt = sm + LD::oBt;
    E* sXt = sm + LD::oXt;
    E* sXwt = sm + LD::oXwt;
    E* sM = sm + LD::oM;
    float* sCs = reinterpret_cast<float*>(smem_raw + LD::nE * sizeof(E));
    float* sDt = sCs + Q;
    int* sSeg = reinterpret_cast<int*>(sDt + Q);
    float* sEo = reinterpret_cast<float*>(sSeg + Q);
    float* sW = sEo + Q;

    const int L = a.L, H = a.H, G = a.G;
    const int nwg = a.B * H;
    const int id = xcd_remap(blockIdx.x, nwg);
    const int b = id / H, h = id % H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;             // lane group (K sub-block / row group)
    const int j16 = lane & 15;            // row/column index inside a tile
    const int p0 = wave * 16;             // this wave's head channels
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float dtb = (a.dt_softplus && a.dt_bias) ? a.dt_bias[h] : 0.0f;
    const int tl = L - 1;                 // last valid token (loads clamp to it)

    const E* xg = static_cast<const E*>(a.x) + (size_t)b * L * a.x_stride + (size_t)h * 64 + p0 + 4 * q4;
    const E* zg = a.z ? static_cast<const E*>(a.z) + (size_t)b * L * a.z_stride + (size_t)h * 64 + p0 + 4 * q4 : nullptr;
    const E* Bg = static_cast<const E*>(a.Bm) + (size_t)b * L * a.B_stride + (size_t)g * N;
    const E* Cg = static_cast<const E*>(a.Cm) + (size_t)b * L * a.C_stride + (size_t)g * N;
    const float* dtg = a.dt + (size_t)b * L * a.dt_stride + h;
    const int32_t* docg = a.doc ? a.doc + (size_t)b * L : nullptr;
    float* yg = a.y + (size_t)b * L * a.y_stride + (size_t)h * 64 + p0 + 4 * q4;
    // Absent optional inputs are replaced, for loading only, by in-bounds rows of
    // x and dt, so that every load stays unconditional; their values are unused.
    const E* zsrc = zg ? zg : xg;
    const int64_t zstride = zg ? a.z_stride : a.x_stride;
    const int32_t* docsrc = docg ? docg : reinterpret_cast<const int32_t*>(a.dt) + (size_t)b * L;

    // ---- global -> registers for the chunk starting at token t0.  Every load
    // is unconditional (rows clamp to the last token) so none of them forces
    // an early wait; rows past the end are zeroed where they are consumed.
    auto load_chunk = [&](int t0, CR& r) {
#pragma unroll
        for (int it = 0; it < CR::NIT; ++it) {
            const int item = min(tid + it * kThreads, CR::NITEMS - 1);
            const int rp = item / CR::CPR, col = item % CR::CPR;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int t = min(t0 + 2 * rp + k, tl);
                r.b[it][k] = *reinterpret_cast<const uint4*>(Bg + (size_t)t * a.B_stride + col * R::VE);
                r.c[it][k] = *reinterpret_cast<const uint4*>(Cg + (size_t)t * a.C_stride + col * R::VE);
            }
        }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int t = min(t0 + 16 * ti + j16, tl);
            r.x[ti] = *reinterpret_cast<const Raw4*>(xg + (size_t)t * a.x_stride);
            r.z[ti] = *reinterpret_cast<const Raw4*>(zsrc + (size_t)t * zstride);
        }
        const int t = min(t0 + lane, tl);
        r.dt = dtg[(size_t)t * a.dt_stride];
        r.d0 = docsrc[t];
        r.d1 = docsrc[t > 0 ? t - 1 : 0];
    };

    // ---- initial state: lane (q4, j16) of n-tile nt holds H[n = 16nt + 4q4 + r][p = p0 + j16]
    f32x4 Hs[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (a.init_state) {
            const float4 v = *reinterpret_cast<const float4*>(
                a.init_state + (((size_t)b * H + h) * 64 + p0 + j16) * N + 16 * nt + 4 * q4);
            Hs[nt] = f32x4{v.x, v.y, v.z, v.w};
        } else {
            Hs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const int nchunks = (L + Q - 1) / Q;
    CR regs;
    if (nchunks > 0) load_chunk(0, regs);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * Q;
        const bool tail = t0 + Q > L;                 // chunk-uniform
        const bool tok_ok = t0 + lane < L;
        // ---- segmented cumulative sum of dt*A (log2 domain), lane = token
        float dtl = a.dt_softplus ? softplus_f(regs.dt + dtb) : regs.dt;
        if (tail && !tok_ok) dtl = 0.0f;
        const int bnd = (docg && tok_ok && t0 + lane > 0 && regs.d0 != regs.d1) ? 1 : 0;
        float cs = dtl * A2;
        int seg = bnd ? lane : -1;           // last document start <= lane inside the chunk
        wave_segscan(cs, bnd, seg);
        const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
        const int last_seg = __builtin_amdgcn_readlane(seg, 63);
        const bool has_bnd = last_seg >= 0;
        const int wseg = has_bnd ? last_seg : 0;   // first token of the chunk's last segment

        // registers of this chunk, kept across the prefetch of the next one
        Raw4 xv[4], zv[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            xv[ti] = regs.x[ti];
            zv[ti] = regs.z[ti];
            if (tail && t0 + 16 * ti + j16 >= L) xv[ti] = R::zero4();
        }

        __syncthreads();   // previous chunk's LDS readers are done

        // ---- stage B (row-major + transposed) and C; rows past the end are zero
#pragma unroll
        for (int it = 0; it < CR::NIT; ++it) {
            const int item = tid + it * kThreads;
            if (item < CR::NITEMS) {
                const int rp = item / CR::CPR, col = item % CR::CPR;
                const int s = 2 * rp, n0 = col * R::VE;
                uint4 b0 = regs.b[it][0], b1 = regs.b[it][1], c0 = regs.c[it][0], c1 = regs.c[it][1];
                if (tail) {
                    const uint4 zz = make_uint4(0, 0, 0, 0);
                    if (t0 + s >= L) { b0 = zz; c0 = zz; }
                    if (t0 + s + 1 >= L) { b1 = zz; c1 = zz; }
                }
                *reinterpret_cast<uint4*>(sB + s * NS + n0) = b0;
                *reinterpret_cast<uint4*>(sB + (s + 1) * NS + n0) = b1;
                *reinterpret_cast<uint4*>(sC + s * NS + n0) = c0;
                *reinterpret_cast<uint4*>(sC + (s + 1) * NS + n0) = c1;
#pragma unroll
                for (int e = 0; e < R::VE; ++e)
                    *reinterpret_cast<typename R::Pair*>(sBt + (n0 + e) * kXS + s) = R::pair(b0, b1, e);
            }
        }
        // ---- this wave's X^T
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int t = 16 * ti + j16;
#pragma unroll
            for (int r = 0; r < 4; ++r) sXt[(p0 + 4 * q4 + r) * kXS + t] = R::raw_el(xv[ti], r);
        }
        // ---- per-token scalars of the chunk
        if (wave == 0) {
            sCs[lane] = cs;
            sDt[lane] = dtl;
            sSeg[lane] = seg < 0 ? 0 : seg;
            // Yoff applies while no document has started in [chunk start, t]
            sEo[lane] = seg < 0 ? fast_exp2(cs) : 0.0f;
            // chunk-state weight: decay to the chunk end, on the last segment only
            sW[lane] = lane >= wseg ? fast_exp2(cs_end - cs) * dtl : 0.0f;
        }
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(t0 + Q, regs);

        // ---- this wave's (w o X)^T (read back only by this wave)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int t = 16 * ti + j16;
            const float w = sW[t];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sXwt[(p0 + 4 * q4 + r) * kXS + t] = R::from_f(w * R::el(xv[ti], r));
        }

        // ---- M^T tiles (this wave's share of the lower triangle)
        for (int k = wave; k < kNumMTiles; k += kWaves) {
            int si, ti;
            mtile(k, si, ti);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nb = 0; nb < NT; nb += 2) {
                const Frag a0 = R::ld(sB + (16 * si + j16) * NS + 16 * nb + 4 * q4);
                const Frag b0 = R::ld(sC + (16 * ti + j16) * NS + 16 * nb + 4 * q4);
                const Frag a1 = nb + 1 < NT ? R::ld(sB + (16 * si + j16) * NS + 16 * (nb + 1) + 4 * q4) : R::zero();
                const Frag b1 = nb + 1 < NT ? R::ld(sC + (16 * ti + j16) * NS + 16 * (nb + 1) + 4 * q4) : R::zero();
                acc = R::mma2(acc, a0, a1, b0, b1);
            }
            // acc[r] = G^T[s = 16si + 4q4 + r][t = 16ti + j16]
            const int t = 16 * ti + j16;
            const float cst = sCs[t];
            const int segt = sSeg[t];
            const float4 css = *reinterpret_cast<const float4*>(sCs + 16 * si + 4 * q4);
            const float4 dts = *reinterpret_cast<const float4*>(sDt + 16 * si + 4 * q4);
            f32x4 m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * si + 4 * q4 + r;
                const bool ok = s <= t && s >= segt;
                m[r] = ok ? acc[r] * fast_exp2(cst - (&css.x)[r]) * (&dts.x)[r] : 0.0f;
            }
            const Frag f = R::from_acc(m);
            *reinterpret_cast<Frag*>(sM + k * 256 + lane * 4) = f;
        }

        // ---- chunk state S = B^T (w o X): lane holds S[n = 16nt + 4q4 + r][p0 + j16]
        f32x4 Sacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; sb += 2) {
                const Frag a0 = R::ld(sBt + (16 * nt + j16) * kXS + 16 * sb + 4 * q4);
                const Frag a1 = R::ld(sBt + (16 * nt + j16) * kXS + 16 * (sb + 1) + 4 * q4);
                const Frag b0 = R::ld(sXwt + (p0 + j16) * kXS + 16 * sb + 4 * q4);
                const Frag b1 = R::ld(sXwt + (p0 + j16) * kXS + 16 * (sb + 1) + 4 * q4);
                acc = R::mma2(acc, a0, a1, b0, b1);
            }
            Sacc[nt] = acc;
        }

        // ---- Yoff^T[p, t] = sum_n H[n, p] C[t, n] for the 4 token tiles
        f32x4 Yoff[4];
        {
            Frag hhi[NT], hlo[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (std::is_same<T, float>::value) {
                    hhi[nt] = R::from_acc(Hs[nt]);
                    hlo[nt] = R::zero();
                } else {
                    hhi[nt] = frag_from_f32(Hs[nt]);
                    f32x4 rem;
                    rem[0] = Hs[nt][0] - bf16_lo(hhi[nt].a);
                    rem[1] = Hs[nt][1] - bf16_hi(hhi[nt].a);
                    rem[2] = Hs[nt][2] - bf16_lo(hhi[nt].b);
                    rem[3] = Hs[nt][3] - bf16_hi(hhi[nt].b);
                    hlo[nt] = frag_from_f32(rem);
                }
            }
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nb = 0; nb < NT; nb += 2) {
                    const Frag c0 = R::ld(sC + (16 * ti + j16) * NS + 16 * nb + 4 * q4);
                    const Frag c1 = nb + 1 < NT ? R::ld(sC + (16 * ti + j16) * NS + 16 * (nb + 1) + 4 * q4) : R::zero();
                    const Frag h1 = nb + 1 < NT ? hhi[nb + 1] : R::zero();
                    acc = R::mma2(acc, hhi[nb], h1, c0, c1);
                    if constexpr (!std::is_same<T, float>::value) {
                        const Frag l1 = nb + 1 < NT ? hlo[nb + 1] : R::zero();
                        acc = R::mma2(acc, hlo[nb], l1, c0, c1);
                    }
                }
                Yoff[ti] = acc;
            }
        }
        __syncthreads();   // all M^T tiles are in LDS

        // ---- Ydiag^T[p, t] = sum_s X^T[p, s] M^T[s, t], then the output
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb <= ti; sb += 2) {
                const Frag a0 = R::ld(sXt + (p0 + j16) * kXS + 16 * sb + 4 * q4);
                const Frag b0 = R::ld(sM + mtile_index(sb, ti) * 256 + lane * 4);
                const bool two = sb + 1 <= ti;
                const Frag a1 = two ? R::ld(sXt + (p0 + j16) * kXS + 16 * (sb + 1) + 4 * q4) : R::zero();
                const Frag b1 = two ? R::ld(sM + mtile_index(sb + 1, ti) * 256 + lane * 4) : R::zero();
                acc = R::mma2(acc, a0, a1, b0, b1);
            }
            // lane holds y[t = 16ti + j16][p = p0 + 4q4 + r]
            const int t = 16 * ti + j16;
            const float eo = sEo[t];
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = fmaf(eo, Yoff[ti][r], acc[r]);
                v = fmaf(Dh, R::el(xv[ti], r), v);
                if (zg) v *= silu_f(R::el(zv[ti], r));
                o[r] = v;
            }
            if (!tail || t0 + t < L)
                *reinterpret_cast<float4*>(yg + (size_t)(t0 + t) * a.y_stride) = make_float4(o[0], o[1], o[2], o[3]);
        }

        // ---- state passing, strictly in chunk order
        const float dec = fast_exp2(cs_end);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Hs[nt][r] = has_bnd ? Sacc[nt][r] : fmaf(dec, Hs[nt][r], Sacc[nt][r]);
    }

    if (a.final_state) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<float4*>(a.final_state + (((size_t)b * H + h) * 64 + p0 + j16) * N + 16 * nt + 4 * q4) =
                make_float4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
    }
}

template <typename T, int N>
hipError_t launch_scan_n(const ScanArgs& a, hipStream_t stream) {
    const size_t lds = Lds<T, N>::bytes;
    static bool attr_set = false;   // raise the dynamic-LDS cap once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_scan_kernel<T, N>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((ssd_scan_kernel<T, N>), dim3(a.B * a.H), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_scan_n<T, 16>(a, stream);
        case 32: return launch_scan_n<T, 32>(a, stream);
        case 64: return launch_scan_n<T, 64>(a, stream);
        case 128: return launch_scan_n<T, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t scan_lds_bytes(int N, int dtype) {
    switch (N) {
        case 16: return dtype == 0 ? Lds<float, 16>::bytes : Lds<uint16_t, 16>::bytes;
        case 32: return dtype == 0 ? Lds<float, 32>::bytes : Lds<uint16_t, 32>::bytes;
        case 64: return dtype == 0 ? Lds<float, 64>::bytes : Lds<uint16_t, 64>::bytes;
        case 128: return dtype == 0 ? Lds<float, 128>::bytes : Lds<uint16_t, 128>::bytes;
    }
    return 0;
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 0 ? launch_scan_t<float>(a, stream) : launch_scan_t<uint16_t>(a, stream);
}

}  // namespace ssd
