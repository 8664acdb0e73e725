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

// MODE kFull: the scan itself.  MODE kStateOnly: the pre-pass of the sequence
// split -- for superchunk k < K-1 of (b, h) it runs the chunk-state recurrence
// from a zero state and stores the local end state and the superchunk's total
// decay (negative if a document starts inside it, i.e. the carried state is
// dropped there) into the workspace.
enum { kFull = 0, kStateOnly = 1 };

// LDS plan (element offsets).  kFull: region R0 holds B row-major while the
// M^T tiles are built, then this wave's (w o X)^T for the chunk state; C,
// B^T, X^T, the M^T tiles, then fp32 per-token scalars.  kStateOnly: B^T,
// (w o X)^T, scalars.
template <typename T, int N, int MODE>
struct Lds {
    using E = typename Tr<T>::E;
    static constexpr int NS = N + kPad;                          // row stride of B and C
    static constexpr size_t r0 = (size_t)Q * NS > (size_t)64 * kXS ? (size_t)Q * NS : (size_t)64 * kXS;
    static constexpr size_t oB = 0;                              // B [Q][NS]      (kFull)
    static constexpr size_t oXwt = MODE == kFull ? 0 : (size_t)N * kXS;   // (wX)^T [64 p][kXS]
    static constexpr size_t oC = r0;                             // C [Q][NS]      (kFull)
    static constexpr size_t oBt = MODE == kFull ? oC + (size_t)Q * NS : 0;  // B^T [N][kXS]
    static constexpr size_t oXt = oBt + (size_t)N * kXS;         // X^T [64 p][kXS] (kFull)
    static constexpr size_t oM = oXt + (size_t)64 * kXS;         // M^T tiles [10][64 lanes][4] (kFull)
    static constexpr size_t nE = MODE == kFull ? oM + (size_t)kNumMTiles * 256 : oXwt + (size_t)64 * kXS;
    // per-token scalars (kFull: cs, dt, segment start, Yoff scale), then the
    // chunk-state weights, one private row per wave
    static constexpr int nScal = (MODE == kFull ? 4 : 0) + kWaves;
    static constexpr size_t bytes = ((nE * sizeof(E) + 15) / 16) * 16 + (size_t)nScal * Q * sizeof(float);
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

template <typename T, int N, int MODE>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(ScanArgs a) {
    using R = Tr<T>;
    using E = typename R::E;
    using Frag = typename R::Frag;
    using Raw4 = typename R::Raw4;
    using LD = Lds<T, N, MODE>;
    using CR = ChunkRegs<T, N>;
    constexpr int NT = N / 16;            // n tiles
    constexpr int NS = LD::NS;
    constexpr bool FULL = MODE == kFull;
    constexpr bool BF16 = !std::is_same<T, float>::value;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    E* sm = reinterpret_cast<E*>(smem_raw);
    E* sB = sm + LD::oB;
    E* sXwt = sm + LD::oXwt;
    E* sC = sm + LD::oC;
    E* sBt = sm + LD::oBt;
    E* sXt = sm + LD::oXt;
    E* sM = sm + LD::oM;
    float* sScal = reinterpret_cast<float*>(smem_raw + ((LD::nE * sizeof(E) + 15) / 16) * 16);
    float* sCs = sScal;
    float* sDt = sScal + Q;
    int* sSeg = reinterpret_cast<int*>(sScal + 2 * Q);
    float* sEo = sScal + 3 * Q;
    float* sW = sScal + (FULL ? 4 : 0) * Q;   // [kWaves][Q]

    const int L = a.L, H = a.H, G = a.G;
    const int KU = FULL ? a.K : a.K - 1;  // superchunks handled by this launch per (b, h)
    const int id = xcd_remap(blockIdx.x, a.B * H * KU);
    const int h = id % H;
    const int k = (id / H) % KU;
    const int b = id / (H * KU);
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
    const int tbeg = k * a.S;
    const int tend = min(tbeg + a.S, L);
    const int tl = tend - 1;              // last token of this unit (loads clamp to it)
    const bool gate = a.z != nullptr;

    // Row bases (uniform) and per-lane element offsets; a chunk's loads are
    // base + t0 * stride (scalar) + lane offset, rows clamped only in the tail.
    const E* xbase = static_cast<const E*>(a.x) + (size_t)b * L * a.x_stride;
    const E* zbase = gate ? static_cast<const E*>(a.z) + (size_t)b * L * a.z_stride : xbase;
    const int64_t zs = gate ? a.z_stride : a.x_stride;
    const E* Bbase = static_cast<const E*>(a.Bm) + (size_t)b * L * a.B_stride;
    const E* Cbase = static_cast<const E*>(a.Cm) + (size_t)b * L * a.C_stride;
    const float* dtbase = a.dt + (size_t)b * L * a.dt_stride;
    const int32_t* docg = a.doc ? a.doc + (size_t)b * L : nullptr;
    // absent doc ids: load (unused) in-bounds words of dt instead, keeping loads unconditional
    const int32_t* docsrc = docg ? docg : reinterpret_cast<const int32_t*>(dtbase);
    const int xcol = h * 64 + p0 + 4 * q4;
    float* yg = a.y + (size_t)b * L * a.y_stride + xcol;

    // Loads: a uniform chunk base (t0 * stride, scalar) plus a 32-bit per-lane
    // byte offset fixed for the whole unit; only a chunk that runs past the
    // unit's end recomputes offsets with rows clamped to its last token.
    constexpr int ES = (int)sizeof(E);
    int bo[CR::NIT];                       // B/C: (row pair, 16-byte column) item of this thread
#pragma unroll
    for (int it = 0; it < CR::NIT; ++it) {
        const int item = min(tid + it * kThreads, CR::NITEMS - 1);
        const int rp = item / CR::CPR, col = item % CR::CPR;
        bo[it] = rp;
        (void)col;
    }
    auto bc_col = [&](int it) { return (min(tid + it * kThreads, CR::NITEMS - 1) % CR::CPR) * R::VE; };
    auto load_chunk = [&](int t0, CR& r) {
        const int lim = tl - t0;                     // last valid row inside the chunk
        const bool clamp = lim < Q - 1;              // uniform
        const char* Bb = reinterpret_cast<const char*>(Bbase + (size_t)t0 * a.B_stride + g * N);
        const char* Cb = reinterpret_cast<const char*>(Cbase + (size_t)t0 * a.C_stride + g * N);
#pragma unroll
        for (int it = 0; it < CR::NIT; ++it) {
            const int col = bc_col(it);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                int row = 2 * bo[it] + kk;
                if (clamp) row = min(row, lim);
                const uint32_t ob = (uint32_t)(row * (int)a.B_stride + col) * ES;
                r.b[it][kk] = *reinterpret_cast<const uint4*>(Bb + ob);
                if (FULL) {
                    const uint32_t oc = (uint32_t)(row * (int)a.C_stride + col) * ES;
                    r.c[it][kk] = *reinterpret_cast<const uint4*>(Cb + oc);
                }
            }
        }
        const char* xb = reinterpret_cast<const char*>(xbase + (size_t)t0 * a.x_stride + xcol);
        const char* zb = reinterpret_cast<const char*>(zbase + (size_t)t0 * zs + xcol);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            int row = 16 * ti + j16;
            if (clamp) row = min(row, lim);
            r.x[ti] = *reinterpret_cast<const Raw4*>(xb + (uint32_t)(row * (int)a.x_stride) * ES);
            if (FULL) r.z[ti] = *reinterpret_cast<const Raw4*>(zb + (uint32_t)(row * (int)zs) * ES);
        }
        int row = lane;
        if (clamp) row = min(row, lim);
        const char* db = reinterpret_cast<const char*>(dtbase + (size_t)t0 * a.dt_stride + h);
        r.dt = *reinterpret_cast<const float*>(db + (uint32_t)(row * (int)a.dt_stride) * 4);
        r.d0 = docsrc[t0 + row];
        r.d1 = docsrc[max(t0 + row - 1, 0)];
    };

    // ---- state at the unit's first token: lane (q4, j16) of n-tile nt holds
    // H[n = 16nt + 4q4 + r][p = p0 + j16].  Superchunk 0 starts from the caller's
    // initial state; superchunk k > 0 folds the pre-pass results of 0..k-1 in
    // order, H = (reset ? 0 : decay * H) + local state.
    f32x4 Hs[NT];
    const size_t st_off = (((size_t)b * H + h) * 64 + p0 + j16) * N + 4 * q4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Hs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (FULL) {
        if (a.init_state) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4 v = *reinterpret_cast<const float4*>(a.init_state + st_off + 16 * nt);
                Hs[nt] = f32x4{v.x, v.y, v.z, v.w};
            }
        }
        for (int j = 0; j < k; ++j) {
            const size_t u = ((size_t)b * H + h) * (a.K - 1) + j;
            const float dj = a.dec[u];
            const float* hl = a.hloc + u * 64 * N + (size_t)(p0 + j16) * N + 4 * q4;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4 v = *reinterpret_cast<const float4*>(hl + 16 * nt);
                Hs[nt][0] = dj < 0.0f ? v.x : fmaf(dj, Hs[nt][0], v.x);
                Hs[nt][1] = dj < 0.0f ? v.y : fmaf(dj, Hs[nt][1], v.y);
                Hs[nt][2] = dj < 0.0f ? v.z : fmaf(dj, Hs[nt][2], v.z);
                Hs[nt][3] = dj < 0.0f ? v.w : fmaf(dj, Hs[nt][3], v.w);
            }
        }
    }
    float log2dec = 0.0f;                 // kStateOnly: sum of the chunks' cs_end
    bool reset = false;                   // kStateOnly: a document starts in the unit

    const int nchunks = (tend - tbeg + Q - 1) / Q;
    CR regs;
    if (nchunks > 0) load_chunk(tbeg, regs);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = tbeg + c * Q;
        const bool tail = t0 + Q > tend;              // chunk-uniform
        const bool tok_ok = t0 + lane < tend;
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
            if (tail && t0 + 16 * ti + j16 >= tend) xv[ti] = R::zero4();
        }
        // chunk-state weight of token `lane`: decay to the chunk end, last segment only
        float* sWw = sW + wave * Q;
        sWw[lane] = lane >= wseg ? fast_exp2(cs_end - cs) * dtl : 0.0f;

        __syncthreads();   // previous chunk's LDS readers are done

        // ---- stage B (row-major + transposed) and C; rows past the end are zero
#pragma unroll
        for (int it = 0; it < CR::NIT; ++it) {
            const int item = tid + it * kThreads;
            if (item < CR::NITEMS) {
                const int rp = item / CR::CPR, col = item % CR::CPR;
                const int s = 2 * rp, n0 = col * R::VE;
                uint4 b0 = regs.b[it][0], b1 = regs.b[it][1];
                uint4 c0 = regs.c[it][0], c1 = regs.c[it][1];
                if (tail) {
                    const uint4 zz = make_uint4(0, 0, 0, 0);
                    if (t0 + s >= tend) { b0 = zz; c0 = zz; }
                    if (t0 + s + 1 >= tend) { b1 = zz; c1 = zz; }
                }
                if (FULL) {
                    *reinterpret_cast<uint4*>(sB + s * NS + n0) = b0;
                    *reinterpret_cast<uint4*>(sB + (s + 1) * NS + n0) = b1;
                    *reinterpret_cast<uint4*>(sC + s * NS + n0) = c0;
                    *reinterpret_cast<uint4*>(sC + (s + 1) * NS + n0) = c1;
                }
#pragma unroll
                for (int e = 0; e < R::VE; ++e)
                    *reinterpret_cast<typename R::Pair*>(sBt + (n0 + e) * kXS + s) = R::pair(b0, b1, e);
            }
        }
        // ---- (w o X)^T (kStateOnly) or X^T (kFull) of this wave's channels
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int t = 16 * ti + j16;
            if (FULL) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sXt[(p0 + 4 * q4 + r) * kXS + t] = R::raw_el(xv[ti], r);
            } else {
                const float w = sWw[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) sXwt[(p0 + 4 * q4 + r) * kXS + t] = R::from_f(w * R::el(xv[ti], r));
            }
        }
        // ---- per-token scalars of the chunk
        if (FULL && wave == 0) {
            sCs[lane] = cs;
            sDt[lane] = dtl;
            sSeg[lane] = seg < 0 ? 0 : seg;
            // Yoff applies while no document has started in [chunk start, t]
            sEo[lane] = seg < 0 ? fast_exp2(cs) : 0.0f;
        }
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(t0 + Q, regs);

        if (FULL) {
            // ---- M^T tiles (this wave's share of the lower triangle)
            for (int kt = wave; kt < kNumMTiles; kt += kWaves) {
                int si, ti;
                mtile(kt, si, ti);
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
                    const bool ok = (si < ti || s <= t) && (!has_bnd || s >= segt);
                    m[r] = ok ? acc[r] * fast_exp2(cst - (&css.x)[r]) * (&dts.x)[r] : 0.0f;
                }
                *reinterpret_cast<Frag*>(sM + kt * 256 + lane * 4) = R::from_acc(m);
            }
            // bf16 (or fp32) copy of the carried state for the C.H contraction
            Frag hf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) hf[nt] = R::from_acc(Hs[nt]);
            __syncthreads();   // all M^T tiles are in LDS; B row-major is no longer read

            // ---- per token tile: Ydiag^T = X^T M^T, Yoff^T = H^T C^T, then the output
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 yd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sb = 0; sb <= ti; sb += 2) {
                    const Frag a0 = R::ld(sXt + (p0 + j16) * kXS + 16 * sb + 4 * q4);
                    const Frag b0 = R::ld(sM + mtile_index(sb, ti) * 256 + lane * 4);
                    const bool two = sb + 1 <= ti;
                    const Frag a1 = two ? R::ld(sXt + (p0 + j16) * kXS + 16 * (sb + 1) + 4 * q4) : R::zero();
                    const Frag b1 = two ? R::ld(sM + mtile_index(sb + 1, ti) * 256 + lane * 4) : R::zero();
                    yd = R::mma2(yd, a0, a1, b0, b1);
                }
                f32x4 yo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nb = 0; nb < NT; nb += 2) {
                    const Frag c0 = R::ld(sC + (16 * ti + j16) * NS + 16 * nb + 4 * q4);
                    const Frag c1 = nb + 1 < NT ? R::ld(sC + (16 * ti + j16) * NS + 16 * (nb + 1) + 4 * q4) : R::zero();
                    const Frag h1 = nb + 1 < NT ? hf[nb + 1] : R::zero();
                    yo = R::mma2(yo, hf[nb], h1, c0, c1);
                }
                // lane holds y[t = 16ti + j16][p = p0 + 4q4 + r]
                const int t = 16 * ti + j16;
                const float eo = sEo[t];
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = fmaf(eo, yo[r], yd[r]);
                    v = fmaf(Dh, R::el(xv[ti], r), v);
                    if (gate) v *= silu_f(R::el(zv[ti], r));
                    o[r] = v;
                }
                if (!tail || t0 + t < tend)
                    *reinterpret_cast<float4*>(yg + (size_t)(t0 + t) * a.y_stride) = make_float4(o[0], o[1], o[2], o[3]);
            }
            // ---- (w o X)^T of this wave's channels, into the B row-major area
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int t = 16 * ti + j16;
                const float w = sWw[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) sB[(p0 + 4 * q4 + r) * kXS + t] = R::from_f(w * R::el(xv[ti], r));
            }
        }

        // ---- chunk state S = B^T (w o X): lane holds S[n = 16nt + 4q4 + r][p0 + j16],
        // then the state passing, strictly in chunk order
        const E* xw = FULL ? sB : sXwt;
        const float dec = fast_exp2(cs_end);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; sb += 2) {
                const Frag a0 = R::ld(sBt + (16 * nt + j16) * kXS + 16 * sb + 4 * q4);
                const Frag a1 = R::ld(sBt + (16 * nt + j16) * kXS + 16 * (sb + 1) + 4 * q4);
                const Frag b0 = R::ld(xw + (p0 + j16) * kXS + 16 * sb + 4 * q4);
                const Frag b1 = R::ld(xw + (p0 + j16) * kXS + 16 * (sb + 1) + 4 * q4);
                acc = R::mma2(acc, a0, a1, b0, b1);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Hs[nt][r] = has_bnd ? acc[r] : fmaf(dec, Hs[nt][r], acc[r]);
        }
        if (!FULL) {
            log2dec += cs_end;
            reset = reset || has_bnd;
        }
    }

    if (FULL) {
        if (a.final_state && k == a.K - 1) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<float4*>(a.final_state + st_off + 16 * nt) =
                    make_float4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
        }
    } else {
        const size_t u = ((size_t)b * H + h) * (a.K - 1) + k;
        float* hl = a.hloc + u * 64 * N + (size_t)(p0 + j16) * N + 4 * q4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<float4*>(hl + 16 * nt) = make_float4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
        if (tid == 0) a.dec[u] = reset ? -1.0f : fast_exp2(log2dec);
    }
}

// ============================================================================
// bf16 kernel: LDS-DMA pipeline.
//
// B, C and this head's X rows of a chunk stream from HBM straight into
// row-major LDS tiles with global_load_lds (16 bytes per lane, lane-linear
// destination), two chunk stages deep: the copy of chunk c+1 is in flight
// while chunk c computes, and no registers or VALU are spent on staging.
// Transposed operands (B^T for the chunk state, X^T and (w o X)^T) come from
// the same row-major tiles through ds_read_b64_tr_b16: in each 16-lane group,
// result lane j element e is element (j mod 4) of source lane 4e + j/4, so a
// lane (q, m) that addresses row 4q + m/4, column 4(m mod 4) of a tile
// receives column m, rows 4q..4q+3 -- exactly the operand fragment of the
// transposed tile.  Two barriers per chunk; per-token scalars are double
// buffered so wave 0 can publish chunk c+1's while others finish chunk c.
// ============================================================================
typedef short v4i16_t __attribute__((ext_vector_type(4)));
#define SSD_LDS __attribute__((address_space(3)))

__device__ __forceinline__ FragBF tr_read(const unsigned char* lds_base, uint32_t byte_off) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSD_LDS v4i16_t*)(lds_base + byte_off));
    FragBF f;
    f.a = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    f.b = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    return f;
}
__device__ __forceinline__ FragBF plain_read(const unsigned char* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return {v.x, v.y};
}
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
    __builtin_amdgcn_global_load_lds(g, (SSD_LDS void*)lds, 16, 0, 0);
}

// XOR swizzle of 16-byte pieces inside a tile row of RB bytes: piece c of row r
// is stored at position c ^ f(r), f(r) = (r / rows-per-256B) mod pieces-per-row.
// Sixteen consecutive rows read at one column then fall on sixteen different
// bank groups (the MFMA fragment reads and the transpose reads both read 16 or
// 4 x 4 rows at one column).  Because 16 / rows-per-256B equals the pieces per
// row, f depends only on the row's position inside its 16-row tile.
template <int RB>
struct Swz {
    static constexpr int CPR = RB / 16;
    static constexpr int RL = RB >= 256 ? 1 : 256 / RB;
    __device__ static int f(int row) { return (row / RL) % CPR; }
    __device__ static uint32_t off(int row, int col) {   // byte offset of element col (multiple of 4) of row
        return (uint32_t)(row * RB + ((((col >> 3) ^ f(row)) << 4) | ((col & 7) * 2)));
    }
};

template <int N, int MODE>
struct LdsBf {
    static constexpr int RB = N * 2;                  // bytes per B / C row
    static constexpr int XB = 128;                    // bytes per X row (64 channels)
    static constexpr int TB = Q * RB;                 // B or C tile
    static constexpr int TX = Q * XB;                 // X tile
    static constexpr bool FULL = MODE == kFull;
    static constexpr int oB = 0, oC = TB, oX = FULL ? 2 * TB : TB;
    static constexpr int STAGE = oX + TX;
    // Copies run NSTAGE-1 chunks ahead; three stages where two workgroups
    // still fit a CU's 160 KiB, else two.
    static constexpr int NSTAGE = (3 * STAGE + (FULL ? kNumMTiles * 512 : 0) + 2560) * 2 <= 163840 ? 3 : 2;
    static constexpr int oM = NSTAGE * STAGE;         // M^T tiles (kFull) [10][64][4] bf16
    static constexpr int oS = oM + (FULL ? kNumMTiles * 256 * 2 : 0);   // scalars [2][5][Q] fp32
    static constexpr int bytes = oS + 2 * 5 * Q * 4;
    // vector-memory instructions one wave issues per chunk: the plain loads
    // (dt, two doc ids, four z rows in kFull) and its share of the copies;
    // the fewest over the four waves, so a wait for "at most this many newer
    // operations outstanding" is never too lenient
    static constexpr int RPI_B = 64 / (RB / 16);
    static constexpr int nB_min = (Q / RPI_B) / kWaves;               // floor: waves that get fewer
    static constexpr int VM_PER_CHUNK = 3 + (FULL ? 4 : 0) + nB_min * (FULL ? 2 : 1) + (Q / 8) / kWaves;
};

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt left at their maximum).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

template <int N, int MODE, bool SP>
__global__ __launch_bounds__(kThreads) void ssd_scan_bf16_kernel(ScanArgs a) {
    using LD = LdsBf<N, MODE>;
    constexpr int NT = N / 16;
    constexpr bool FULL = MODE == kFull;
    constexpr int RB = LD::RB, XB = LD::XB;
    constexpr int CPR_B = RB / 16, RPI_B = 64 / CPR_B;    // 16-byte pieces per B row, rows per DMA
    constexpr int RPI_X = 64 / (XB / 16);                  // 8 rows per X DMA
    using SB = Swz<RB>;
    using SX = Swz<XB>;

    extern __shared__ __align__(16) unsigned char smem[];
    float* scal = reinterpret_cast<float*>(smem + LD::oS);   // [2][5][Q]: cs, dt, seg, eo, w

    const int L = a.L, H = a.H, G = a.G;
    const int KU = FULL ? a.K : a.K - 1;
    const int id = xcd_remap(blockIdx.x, a.B * H * KU);
    const int h = id % H;
    const int k = (id / H) % KU;
    const int b = id / (H * KU);
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int j16 = lane & 15;
    const int p0 = wave * 16;
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float dtb = (a.dt_softplus && a.dt_bias) ? a.dt_bias[h] : 0.0f;
    const int tbeg = k * a.S;
    const int tend = min(tbeg + a.S, L);
    const int tl = tend - 1;
    const bool gate = a.z != nullptr;

    const uint16_t* xbase = static_cast<const uint16_t*>(a.x) + (size_t)b * L * a.x_stride + (size_t)h * 64;
    const uint16_t* zbase = gate ? static_cast<const uint16_t*>(a.z) + (size_t)b * L * a.z_stride + (size_t)h * 64 : xbase;
    const int64_t zs = gate ? a.z_stride : a.x_stride;
    const uint16_t* Bbase = static_cast<const uint16_t*>(a.Bm) + (size_t)b * L * a.B_stride + (size_t)g * N;
    const uint16_t* Cbase = static_cast<const uint16_t*>(a.Cm) + (size_t)b * L * a.C_stride + (size_t)g * N;
    const float* dtbase = a.dt + (size_t)b * L * a.dt_stride + h;
    const int32_t* docg = a.doc ? a.doc + (size_t)b * L : nullptr;
    const int32_t* docsrc = docg ? docg : reinterpret_cast<const int32_t*>(a.dt) + (size_t)b * L;
    float* yg = a.y + (size_t)b * L * a.y_stride + h * 64 + p0 + 4 * q4;

    // ---- chunk t0 -> LDS stage st (DMA) and the per-lane registers (dt, doc, z);
    // register sets rotate with the stages (set s holds chunk c with c % NSTAGE == s)
    constexpr int NSTAGE = LD::NSTAGE;
    float r_dt[NSTAGE];
    int r_d0[NSTAGE], r_d1[NSTAGE];
    uint2 r_z[NSTAGE][4];
    // Addresses: a uniform chunk base (t0 * stride, scalar) plus a 32-bit
    // per-lane byte offset of row * stride (rows clamp to the unit's end).
    const int Bs = (int)a.B_stride, Cs = (int)a.C_stride, Xs = (int)a.x_stride, Zs = (int)zs, Ds = (int)a.dt_stride;
    auto issue_chunk = [&](int t0, int st, float& o_dt, int& o_d0, int& o_d1, uint2* o_z) {
        const int lim = tl - t0;
        unsigned char* base = smem + st * LD::STAGE;
        const char* Bc = reinterpret_cast<const char*>(Bbase + (size_t)t0 * a.B_stride);
        const char* Cc = reinterpret_cast<const char*>(Cbase + (size_t)t0 * a.C_stride);
        const char* Xc = reinterpret_cast<const char*>(xbase + (size_t)t0 * a.x_stride);
        // plain loads first, then (after a compiler fence) the copies, so the
        // copies of a chunk are the newest vector-memory operations it issues
        const int rowl = min(lane, lim);
        o_dt = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(dtbase + (size_t)t0 * a.dt_stride) +
                                               (uint32_t)(rowl * Ds) * 4);
        o_d0 = docsrc[t0 + rowl];
        o_d1 = docsrc[max(t0 + rowl - 1, 0)];
        if (FULL) {
            const char* Zc = reinterpret_cast<const char*>(zbase + (size_t)t0 * zs + p0 + 4 * q4);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int row = min(16 * ti + j16, lim);
                o_z[ti] = *reinterpret_cast<const uint2*>(Zc + (uint32_t)(row * Zs) * 2);
            }
        }
        __asm__ volatile("" ::: "memory");
        for (int ins = wave; ins < Q / RPI_B; ins += kWaves) {
            const int r = ins * RPI_B + lane / CPR_B;            // tile row of this lane's slot
            const int col = (((lane % CPR_B) ^ SB::f(r))) * 8;   // piece stored in that slot
            const int row = min(r, lim);
            dma16(Bc + (uint32_t)(row * Bs + col) * 2, base + LD::oB + ins * 1024);
            if (FULL) dma16(Cc + (uint32_t)(row * Cs + col) * 2, base + LD::oC + ins * 1024);
        }
        for (int ins = wave; ins < Q / RPI_X; ins += kWaves) {
            const int r = ins * RPI_X + lane / (XB / 16);
            const int col = ((lane % (XB / 16)) ^ SX::f(r)) * 8;
            const int row = min(r, lim);
            dma16(Xc + (uint32_t)(row * Xs + col) * 2, base + LD::oX + ins * 1024);
        }
        __asm__ volatile("" ::: "memory");
    };

    // ---- initial state (see the generic kernel)
    f32x4 Hs[NT];
    const size_t st_off = (((size_t)b * H + h) * 64 + p0 + j16) * N + 4 * q4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Hs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (FULL) {
        if (a.init_state) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4 v = *reinterpret_cast<const float4*>(a.init_state + st_off + 16 * nt);
                Hs[nt] = f32x4{v.x, v.y, v.z, v.w};
            }
        }
        for (int j = 0; j < k; ++j) {
            const size_t u = ((size_t)b * H + h) * (a.K - 1) + j;
            const float dj = a.dec[u];
            const float* hl = a.hloc + u * 64 * N + (size_t)(p0 + j16) * N + 4 * q4;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4 v = *reinterpret_cast<const float4*>(hl + 16 * nt);
                Hs[nt][0] = dj < 0.0f ? v.x : fmaf(dj, Hs[nt][0], v.x);
                Hs[nt][1] = dj < 0.0f ? v.y : fmaf(dj, Hs[nt][1], v.y);
                Hs[nt][2] = dj < 0.0f ? v.z : fmaf(dj, Hs[nt][2], v.z);
                Hs[nt][3] = dj < 0.0f ? v.w : fmaf(dj, Hs[nt][3], v.w);
            }
        }
    }
    float log2dec = 0.0f;
    bool reset = false;

    const int nchunks = (tend - tbeg + Q - 1) / Q;
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j)
        if (j < nchunks) issue_chunk(tbeg + j * Q, j, r_dt[j], r_d0[j], r_d1[j], r_z[j]);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = tbeg + c * Q;
        const int st = c % NSTAGE;
        const unsigned char* sB = smem + st * LD::STAGE + LD::oB;
        const unsigned char* sC = smem + st * LD::STAGE + LD::oC;
        const unsigned char* sX = smem + st * LD::STAGE + LD::oX;
        float* sc = scal + (c & 1) * 5 * Q;        // this chunk's scalars
        const bool tok_ok = t0 + lane < tend;
        float c_dt = r_dt[0];
        int c_d0 = r_d0[0], c_d1 = r_d1[0];
        uint2 z_cur[4] = {r_z[0][0], r_z[0][1], r_z[0][2], r_z[0][3]};
#pragma unroll
        for (int j = 1; j < NSTAGE; ++j)
            if (st == j) {
                c_dt = r_dt[j];
                c_d0 = r_d0[j];
                c_d1 = r_d1[j];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) z_cur[ti] = r_z[j][ti];
            }
        // ---- segmented cumulative sum of dt*A (log2 domain), lane = token
        float dtl = c_dt;
        if (SP) dtl = softplus_f(dtl + dtb);
        if (!tok_ok) dtl = 0.0f;
        const int bnd = (docg && tok_ok && t0 + lane > 0 && c_d0 != c_d1) ? 1 : 0;
        float cs = dtl * A2;
        int seg = bnd ? lane : -1;
        wave_segscan(cs, bnd, seg);
        const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
        const int last_seg = __builtin_amdgcn_readlane(seg, 63);
        const bool has_bnd = last_seg >= 0;
        const int wseg = has_bnd ? last_seg : 0;
        if (wave == 0) {
            sc[lane] = cs;
            sc[Q + lane] = dtl;
            reinterpret_cast<int*>(sc)[2 * Q + lane] = seg < 0 ? 0 : seg;
            sc[3 * Q + lane] = seg < 0 ? fast_exp2(cs) : 0.0f;
            sc[4 * Q + lane] = lane >= wseg ? fast_exp2(cs_end - cs) * dtl : 0.0f;
        }
        // this wave's copies of chunk c have landed: only chunk c+1's operations
        // (issued after them, NSTAGE = 3) or nothing (last chunk, NSTAGE = 2) may
        // still be outstanding; newer stores only make the wait stricter
        if (NSTAGE == 3 && c + 1 < nchunks)
            wait_vmcnt<LD::VM_PER_CHUNK>();
        else
            wait_vmcnt<0>();
        __syncthreads();                 // chunk c tiles + scalars visible; chunk c-1 readers done
        {
            const int cn = c + NSTAGE - 1;    // chunk whose copies start now, into the stage chunk c-1 used
            const int sn = cn % NSTAGE;
            if (cn < nchunks) {
#pragma unroll
                for (int j = 0; j < NSTAGE; ++j)
                    if (sn == j) issue_chunk(tbeg + cn * Q, j, r_dt[j], r_d0[j], r_d1[j], r_z[j]);
            }
        }

        if (FULL) {
            unsigned char* sM = smem + LD::oM;
            // ---- M^T tiles: G^T = B C^T (plain row reads), decay, mask -> bf16 fragments
            for (int kt = wave; kt < kNumMTiles; kt += kWaves) {
                int si, ti;
                mtile(kt, si, ti);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nb = 0; nb < NT; nb += 2) {
                    const FragBF a0 = plain_read(sB + SB::off(16 * si + j16, 16 * nb + 4 * q4));
                    const FragBF b0 = plain_read(sC + SB::off(16 * ti + j16, 16 * nb + 4 * q4));
                    FragBF a1 = {0u, 0u}, b1 = {0u, 0u};
                    if (nb + 1 < NT) {
                        a1 = plain_read(sB + SB::off(16 * si + j16, 16 * (nb + 1) + 4 * q4));
                        b1 = plain_read(sC + SB::off(16 * ti + j16, 16 * (nb + 1) + 4 * q4));
                    }
                    acc = mma_bf16(acc, a0, a1, b0, b1);
                }
                const int t = 16 * ti + j16;
                const float cst = sc[t];
                const int segt = reinterpret_cast<const int*>(sc)[2 * Q + t];
                const float4 css = *reinterpret_cast<const float4*>(sc + 16 * si + 4 * q4);
                const float4 dts = *reinterpret_cast<const float4*>(sc + Q + 16 * si + 4 * q4);
                f32x4 m;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * si + 4 * q4 + r;
                    const bool ok = (si < ti || s <= t) && (!has_bnd || s >= segt);
                    m[r] = ok ? acc[r] * fast_exp2(cst - (&css.x)[r]) * (&dts.x)[r] : 0.0f;
                }
                *reinterpret_cast<FragBF*>(sM + (kt * 256 + lane * 4) * 2) = frag_from_f32(m);
            }
            FragBF hf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) hf[nt] = frag_from_f32(Hs[nt]);
            __syncthreads();   // all M^T tiles are in LDS

            // ---- per token tile: Ydiag^T = X^T M^T, Yoff^T = H^T C^T, output
            float* yc = yg + (size_t)t0 * a.y_stride;
            const int Ys = (int)a.y_stride;
            // f of the transpose-read rows does not depend on the 16-row block sb
            const uint32_t xtr = SX::off(4 * q4 + j16 / 4, p0 + 4 * (j16 % 4));
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 yd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sb = 0; sb <= ti; sb += 2) {
                    const FragBF a0 = tr_read(sX, xtr + 16 * sb * XB);
                    const FragBF b0 = plain_read(sM + (mtile_index(sb, ti) * 256 + lane * 4) * 2);
                    FragBF a1 = {0u, 0u}, b1 = {0u, 0u};
                    if (sb + 1 <= ti) {
                        a1 = tr_read(sX, xtr + 16 * (sb + 1) * XB);
                        b1 = plain_read(sM + (mtile_index(sb + 1, ti) * 256 + lane * 4) * 2);
                    }
                    yd = mma_bf16(yd, a0, a1, b0, b1);
                }
                f32x4 yo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nb = 0; nb < NT; nb += 2) {
                    const FragBF c0 = plain_read(sC + SB::off(16 * ti + j16, 16 * nb + 4 * q4));
                    FragBF c1 = {0u, 0u}, h1 = {0u, 0u};
                    if (nb + 1 < NT) {
                        c1 = plain_read(sC + SB::off(16 * ti + j16, 16 * (nb + 1) + 4 * q4));
                        h1 = hf[nb + 1];
                    }
                    yo = mma_bf16(yo, hf[nb], h1, c0, c1);
                }
                const int t = 16 * ti + j16;
                const float eo = sc[3 * Q + t];
                const uint2 xr = *reinterpret_cast<const uint2*>(sX + SX::off(t, p0 + 4 * q4));
                const float xs[4] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y)};
                const float zsv[4] = {bf16_lo(z_cur[ti].x), bf16_hi(z_cur[ti].x), bf16_lo(z_cur[ti].y),
                                      bf16_hi(z_cur[ti].y)};
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = fmaf(eo, yo[r], yd[r]);
                    v = fmaf(Dh, xs[r], v);
                    if (gate) v *= silu_f(zsv[r]);
                    o[r] = v;
                }
                if (t0 + t < tend)
                    *reinterpret_cast<float4*>(reinterpret_cast<char*>(yc) + (uint32_t)(t * Ys) * 4) =
                        make_float4(o[0], o[1], o[2], o[3]);
            }
        }

        // ---- chunk state S = B^T (w o X) from the row-major tiles via transpose reads
        FragBF xw[4];
        {
            const uint32_t xtr = SX::off(4 * q4 + j16 / 4, p0 + 4 * (j16 % 4));
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const FragBF xf = tr_read(sX, xtr + 16 * sb * XB);
                const float4 w = *reinterpret_cast<const float4*>(sc + 4 * Q + 16 * sb + 4 * q4);
                xw[sb].a = pack_bf16x2(w.x * bf16_lo(xf.a), w.y * bf16_hi(xf.a));
                xw[sb].b = pack_bf16x2(w.z * bf16_lo(xf.b), w.w * bf16_hi(xf.b));
            }
        }
        const float dec = fast_exp2(cs_end);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint32_t btr = SB::off(4 * q4 + j16 / 4, 16 * nt + 4 * (j16 % 4));
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; sb += 2) {
                const FragBF a0 = tr_read(sB, btr + 16 * sb * RB);
                const FragBF a1 = tr_read(sB, btr + 16 * (sb + 1) * RB);
                acc = mma_bf16(acc, a0, a1, xw[sb], xw[sb + 1]);
            }
            if (has_bnd) {
                Hs[nt] = acc;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) Hs[nt][r] = fmaf(dec, Hs[nt][r], acc[r]);
            }
        }
        if (!FULL) {
            log2dec += cs_end;
            reset = reset || has_bnd;
        }
    }

    if (FULL) {
        if (a.final_state && k == a.K - 1) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<float4*>(a.final_state + st_off + 16 * nt) =
                    make_float4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
        }
    } else {
        const size_t u = ((size_t)b * H + h) * (a.K - 1) + k;
        float* hl = a.hloc + u * 64 * N + (size_t)(p0 + j16) * N + 4 * q4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<float4*>(hl + 16 * nt) = make_float4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
        if (tid == 0) a.dec[u] = reset ? -1.0f : fast_exp2(log2dec);
    }
}

template <int N, int MODE, bool SP>
hipError_t launch_scan_bf16_sp(const ScanArgs& a, int units, hipStream_t stream) {
    const size_t lds = LdsBf<N, MODE>::bytes;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_scan_bf16_kernel<N, MODE, SP>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((ssd_scan_bf16_kernel<N, MODE, SP>), dim3(units), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}
template <int N, int MODE>
hipError_t launch_scan_bf16_mode(const ScanArgs& a, int units, hipStream_t stream) {
    return a.dt_softplus ? launch_scan_bf16_sp<N, MODE, true>(a, units, stream)
                         : launch_scan_bf16_sp<N, MODE, false>(a, units, stream);
}

template <typename T, int N, int MODE>
hipError_t launch_scan_mode(const ScanArgs& a, int units, hipStream_t stream) {
    const size_t lds = Lds<T, N, MODE>::bytes;
    static bool attr_set = false;   // raise the dynamic-LDS cap once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_scan_kernel<T, N, MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((ssd_scan_kernel<T, N, MODE>), dim3(units), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T, int N>
hipError_t launch_scan_n(const ScanArgs& a, hipStream_t stream) {
    const int bh = a.B * a.H;
    constexpr bool bf = !std::is_same<T, float>::value;
    if (a.K > 1) {
        hipError_t e = bf ? launch_scan_bf16_mode<N, kStateOnly>(a, bh * (a.K - 1), stream)
                          : launch_scan_mode<T, N, kStateOnly>(a, bh * (a.K - 1), stream);
        if (e != hipSuccess) return e;
    }
    return bf ? launch_scan_bf16_mode<N, kFull>(a, bh * a.K, stream) : launch_scan_mode<T, N, kFull>(a, bh * a.K, stream);
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
        case 16: return dtype == 0 ? Lds<float, 16, kFull>::bytes : Lds<uint16_t, 16, kFull>::bytes;
        case 32: return dtype == 0 ? Lds<float, 32, kFull>::bytes : Lds<uint16_t, 32, kFull>::bytes;
        case 64: return dtype == 0 ? Lds<float, 64, kFull>::bytes : Lds<uint16_t, 64, kFull>::bytes;
        case 128: return dtype == 0 ? Lds<float, 128, kFull>::bytes : Lds<uint16_t, 128, kFull>::bytes;
    }
    return 0;
}

// Sequence split: enough (b, h, superchunk) units to give every CU several
// workgroups, with superchunks of at least 8 chunks.  K = 1 when the (b, h)
// pairs alone already fill the device.
void scan_split(int B, int L, int H, int& K, int& S) {
    constexpr long kTargetUnits = 1024;   // 4 workgroups per CU on 256 CUs
    constexpr int kMinChunks = 8;
    const long bh = (long)B * H;
    const int nch = (L + Q - 1) / Q;
    int k = 1;
    while (bh * k < kTargetUnits && nch / (2 * k) >= kMinChunks) k *= 2;
    const int per = (nch + k - 1) / k;           // chunks per superchunk
    K = (nch + per - 1) / per;
    S = per * Q;
    if (K < 1) { K = 1; S = Q; }
}

size_t scan_workspace_bytes(int B, int L, int H, int P, int N) {
    int K, S;
    scan_split(B, L, H, K, S);
    if (K <= 1) return 0;
    const size_t u = (size_t)B * H * (K - 1);
    return u * (size_t)P * N * sizeof(float) + ((u * sizeof(float) + 255) / 256) * 256;
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 0 ? launch_scan_t<float>(a, stream) : launch_scan_t<uint16_t>(a, stream);
}

}  // namespace ssd
