// scan.hip -- ssd_chunk_scan_fwd: the Mamba-2 SSD selective scan on gfx950.
//
// Recurrence (per batch row b, head h in group g):
//     h_t = exp(dt_t A_h) h_{t-1} + dt_t B_t x_t^T,   y_t = (C_t . h_t + D_h x_t) silu(z_t)
// evaluated in chunks of Q = 64 tokens with the dual (quadratic) form inside
// a chunk and the state passed between chunks (chunk size 64: the
// mojolearn.Mamba3Block description; the layer itself: the Codestral-Mamba
// port header and the Mini-K3-1H card).  Per chunk c with tokens t, s in
// [0, 64) (cs = log2-domain cumulative sum of dt A, restarted at every
// document start inside the chunk):
//   G^T[s,t]  = B_s . C_t                       (MFMA, K = N; 10 lower tiles)
//   M^T[s,t]  = G^T[s,t] 2^(cs_t - cs_s) dt_s    for seg(t) <= s <= t, else 0
//   Ydiag^T   = X^T M^T                          (MFMA, K = s)
//   Yoff^T    = H_prev^T C^T                     (MFMA, K = N)
//   S         = B^T (w o X),  w_s = 2^(cs_end - cs_s) dt_s on the last segment
//   y_t       = Ydiag + [t in a carried segment] 2^(cs_t) Yoff + D x_t, gated
//   H         = chunk holds a boundary ? S : 2^(cs_end) H_prev + S
// Every document mask is a select (or a multiply by exactly zero of a finite
// value), so tokens of a later document are bit-for-bit independent of
// (finite) earlier-document inputs.  The pairwise decay is built from the
// difference cs_t - cs_s (the two sums alone can reach hundreds in magnitude
// within a chunk).
//
// Kernels:
//   ssd_scan_kernel<float, N, MODE>  fp32 inputs: one (b, h) per workgroup,
//       register-prefetch staging, operands split into bf16 high and low
//       halves in LDS and multiplied on the bf16 MFMA (three products per
//       tile); MODE kStateOnly is its pre-pass.
//   ssd_scan_bf16_kernel<N, SP, HPW> bf16 inputs: HPW heads of one B/C group
//       per workgroup, every per-chunk input staged by LDS DMA, bf16 MFMA.
//   ssd_scan_state_kernel<...>       bf16 state-only pre-pass of the split.
// Sequence split: with a workspace, each sequence may be cut into K
// superchunks; a state-only pre-pass stores each superchunk's local end state
// and total decay, and the full pass folds the preceding ones into its
// starting state.  Without a workspace the chunks are walked strictly in
// order, so a prefill split at a multiple of 64 tokens reproduces one call
// bit for bit.
//
// All contractions are 16x16 MFMA tiles whose accumulator layout doubles as
// the next contraction's operand layout (see ssd_device.hpp), so G^T feeds
// the Y contraction and H feeds the C.H contraction without any shuffle.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../../include/ssd.h"
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
template <> struct Tr<float> {             // fp32 storage (register side of the generic kernel)
    using E = float;
    using Raw4 = float4;
    static constexpr int VE = 4;
    __device__ static float el(Raw4 v, int r) { return (&v.x)[r]; }
    __device__ static Raw4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

// Tiles of the lower triangle, dealt round-robin to the waves: tile k -> (si, ti).
// Order: by token tile ti, then si -- (0,0) (0,1) (1,1) (0,2) (1,2) (2,2) (0,3)
// (1,3) (2,3) (3,3) -- so the two tiles (sb, ti), (sb+1, ti) an output tile
// reads together sit next to each other.  The table lives in two immediates
// (4 bits per tile) so no memory is touched.
__device__ __forceinline__ void mtile(int k, int& si, int& ti) {
    constexpr unsigned long long kS = 0x3210210100ull;   // si of tile k in nibble k
    constexpr unsigned long long kT = 0x3333222110ull;   // ti of tile k in nibble k
    si = (int)((kS >> (4 * k)) & 0xF);
    ti = (int)((kT >> (4 * k)) & 0xF);
}
__device__ __forceinline__ int mtile_index(int si, int ti) { return ti * (ti + 1) / 2 + si; }

// Byte offset of a lane's row inside a chunk: row < 64 and a row stride of at
// most 2^22 elements (the entry points refuse longer rows) keep both factors
// below 2^24 and the product below 2^32, so the full-rate 24-bit multiplier
// gives it exactly (a 32-bit multiply issues at a quarter of the rate).
// (The empty asm keeps the compiler from folding the scale into the multiply's
// operands, which turns it back into a 32-bit multiply.)
__device__ __forceinline__ uint32_t row_bytes(int row, int stride, int col, int esize) {
    uint32_t m = __umul24((uint32_t)row, (uint32_t)stride);
    asm("" : "+v"(m));
    return (m + (uint32_t)col) * (uint32_t)esize;
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

// LDS plan of the fp32 kernel, in fp32 slots; every matrix region is split
// (Split4: the hi plane, then the lo plane, in the region's byte size).
// B and C row-major [Q][NS] for the group of the workgroup's HPW heads; per
// head a block of X row-major [Q][kXS] -- each wave's 16 columns are later
// overwritten by its w o X -- and (kFull) the head's M^T tiles.  B^T, X^T
// and (w o X) operands come from the row-major planes through transposed
// reads.  Then fp32 scalars: per head (kFull)
// cs, dt, segment start and the Yoff scale [Q] each, then per wave its
// chunk-state weights [Q].  kStateOnly: B and the (w o X)^T blocks only.
template <int N, int MODE, int HPW>
struct Lds {
    static constexpr bool FULL = MODE == kFull;
    static constexpr int NS = N + kPad;                          // row stride of B and C
    static constexpr int cB = Q * NS, cX = 64 * kXS, cM = kNumMTiles * 256;
    static constexpr size_t oB = 0;
    static constexpr size_t oC = cB;                             // (kFull)
    static constexpr size_t oH = (FULL ? 2 : 1) * (size_t)cB;   // first head block
    static constexpr size_t HB = cX + (FULL ? cM : 0);          // slots per head block
    static constexpr size_t nE = oH + HPW * HB;
    static constexpr int NW = 4 * HPW;
    static constexpr int nScal = (FULL ? 4 * HPW : 0) + NW;
    static constexpr size_t bytes = ((nE * 4 + 15) / 16) * 16 + (size_t)nScal * Q * sizeof(float);
};

template <int N, int HPW>
struct ChunkRegs {
    static constexpr int CPR = N * 4 / 16;                       // 16-byte pieces per B/C row
    static constexpr int NITEMS = 32 * CPR;                      // (row pair, piece) items
    static constexpr int NIT = (NITEMS + 256 * HPW - 1) / (256 * HPW);
    uint4 b[NIT][2], c[NIT][2];
    float4 x[4], z[4];
    float dt;
    int d0, d1;       // document id of the token and of the one before it
};

// fp32 scan: HPW heads of one B/C group per workgroup (4 waves per head,
// wave w -> head w / 4, channels 16 (w mod 4) .. +16), one superchunk of one
// batch row; the next chunk's inputs are prefetched into registers while the
// current one is computed.  B and C are staged (split into bf16 halves) once
// for the HPW heads and each G^T tile is built once and turned into every
// head's M^T tile.  Barriers wait for LDS traffic only, so the register
// prefetch stays in flight across them (the compiler waits for each load
// before its first use).  MODE kFull: the scan itself.  MODE kStateOnly: the
// pre-pass of the sequence split -- for superchunk k < K-1 it runs the
// chunk-state recurrence from a zero state and stores the local end state and
// the superchunk's total decay (negative if a document starts inside it, i.e.
// the carried state is dropped there) into the workspace.
template <typename T, int N, int MODE, int HPW>
__global__ __launch_bounds__(256 * HPW) void ssd_scan_kernel(ScanArgs a) {
    using LD = Lds<N, MODE, HPW>;
    using CR = ChunkRegs<N, HPW>;
    constexpr int NT = N / 16;            // n tiles
    constexpr int NS = LD::NS;
    constexpr int NW = LD::NW;
    constexpr int NTH = 256 * HPW;
    constexpr bool FULL = MODE == kFull;
    static_assert(std::is_same<T, float>::value, "the generic kernel takes fp32 inputs");
    static_assert(LD::bytes <= 163840, "LDS plan exceeds a CU");

    extern __shared__ __align__(16) unsigned char smem_raw[];
    // split regions (see Split4): base of the hi plane and the region's slot count
    auto plane = [&](size_t off) { return reinterpret_cast<uint16_t*>(smem_raw + off * 4); };
    constexpr int cB = LD::cB, cX = LD::cX, cM = LD::cM;
    uint16_t* sB = plane(LD::oB);
    uint16_t* sC = plane(LD::oC);

    const int L = a.L, H = a.H, G = a.G;
    const int HQ = H / HPW;
    const int KU = FULL ? a.K : a.K - 1;  // superchunks handled by this launch per (b, head group)
    const int id = xcd_remap(blockIdx.x, a.B * HQ * KU);
    const int hq = id % HQ;
    const int k = (id / HQ) % KU;
    const int b = id / (HQ * KU);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hh = wave >> 2;             // head of this wave within the workgroup
    const int h = hq * HPW + hh;
    const int g = (hq * HPW) / (H / G);
    const int q4 = lane >> 4;             // lane group (K sub-block / row group)
    const int j16 = lane & 15;            // row/column index inside a tile
    const int p0 = (wave & 3) * 16;       // this wave's head channels
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float dtb = (a.dt_softplus && a.dt_bias) ? a.dt_bias[h] : 0.0f;
    const int tbeg = k * a.S;
    const int tend = min(tbeg + a.S, L);
    const int tl = tend - 1;              // last token of this unit (loads clamp to it)
    const bool gate = a.z != nullptr;

    uint16_t* sX = plane(LD::oH + hh * LD::HB);            // this head's X / (w o X) rows
    uint16_t* sM = plane(LD::oH + hh * LD::HB + cX);       // this head's M^T tiles (kFull)
    float* sScal = reinterpret_cast<float*>(smem_raw + ((LD::nE * 4 + 15) / 16) * 16);
    float* sHd = sScal + (FULL ? 4 * Q * hh : 0);          // this head's scalars (kFull)
    float* sCs = sHd;
    float* sDt = sHd + Q;
    int* sSeg = reinterpret_cast<int*>(sHd + 2 * Q);
    float* sEo = sHd + 3 * Q;
    float* sWw = sScal + (FULL ? 4 * HPW : 0) * Q + wave * Q;   // this wave's chunk-state weights

    // Row bases (uniform) and per-lane element offsets; a chunk's loads are
    // base + t0 * stride (scalar) + lane offset, rows clamped only in the tail.
    const float* xbase = static_cast<const float*>(a.x) + (size_t)b * a.Lb * a.x_stride;
    const float* zbase = gate ? static_cast<const float*>(a.z) + (size_t)b * a.Lb * a.z_stride : xbase;
    const int64_t zs = gate ? a.z_stride : a.x_stride;
    const float* Bbase = static_cast<const float*>(a.Bm) + (size_t)b * a.Lb * a.B_stride;
    const float* Cbase = static_cast<const float*>(a.Cm) + (size_t)b * a.Lb * a.C_stride;
    const float* dtbase = a.dt + (size_t)b * a.Lb * a.dt_stride;
    const int32_t* docg = a.doc ? a.doc + (size_t)b * a.Lb : nullptr;
    // absent doc ids: load (unused) in-bounds words of dt instead, keeping loads unconditional
    const int32_t* docsrc = docg ? docg : reinterpret_cast<const int32_t*>(dtbase);
    const int xcol = h * 64 + p0 + 4 * q4;
    float* yg = a.y + (size_t)b * a.Lb * a.y_stride + xcol;

    auto bc_item = [&](int it) { return min(tid + it * NTH, CR::NITEMS - 1); };
    // B, C, dt and the doc ids of the chunk at t0 (x and z: load_xz)
    auto load_bc = [&](int t0, CR& r) {
        const int lim = tl - t0;                     // last valid row inside the chunk
        const bool clamp = lim < Q - 1;              // uniform
        const char* Bb = reinterpret_cast<const char*>(Bbase + (size_t)t0 * a.B_stride + g * N);
        const char* Cb = reinterpret_cast<const char*>(Cbase + (size_t)t0 * a.C_stride + g * N);
#pragma unroll
        for (int it = 0; it < CR::NIT; ++it) {
            const int item = bc_item(it);
            const int rp = item / CR::CPR, col = (item % CR::CPR) * 4;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                int row = 2 * rp + kk;
                if (clamp) row = min(row, lim);
                const uint32_t ob = row_bytes(row, (int)a.B_stride, col, 4);
                r.b[it][kk] = *reinterpret_cast<const uint4*>(Bb + ob);
                if (FULL) {
                    const uint32_t oc = row_bytes(row, (int)a.C_stride, col, 4);
                    r.c[it][kk] = *reinterpret_cast<const uint4*>(Cb + oc);
                }
            }
        }
        int row = lane;
        if (clamp) row = min(row, lim);
        const char* db = reinterpret_cast<const char*>(dtbase + (size_t)t0 * a.dt_stride + h);
        r.dt = *reinterpret_cast<const float*>(db + row_bytes(row, (int)a.dt_stride, 0, 4));
        r.d0 = docsrc[t0 + row];
        r.d1 = docsrc[max(t0 + row - 1, 0)];
    };
    // this wave's x (and z) rows of the chunk at t0
    auto load_xz = [&](int t0, CR& r) {
        const int lim = tl - t0;
        const bool clamp = lim < Q - 1;
        const char* xb = reinterpret_cast<const char*>(xbase + (size_t)t0 * a.x_stride + xcol);
        const char* zb = reinterpret_cast<const char*>(zbase + (size_t)t0 * zs + xcol);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            int row = 16 * ti + j16;
            if (clamp) row = min(row, lim);
            r.x[ti] = *reinterpret_cast<const float4*>(xb + row_bytes(row, (int)a.x_stride, 0, 4));
            if (FULL) r.z[ti] = *reinterpret_cast<const float4*>(zb + row_bytes(row, (int)zs, 0, 4));
        }
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
        const float* h_init = a.K > 1 ? a.h0 : a.init_state;
        if (h_init) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4 v = *reinterpret_cast<const float4*>(h_init + st_off + 16 * nt);
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

    // byte offsets of this lane's transposed reads in the hi planes (the lo
    // plane is the region's slot count * 2 bytes on): B^T of n tile nt, token
    // block sb at btr + (16 sb NS + 16 nt) * 2; the wave's X^T / (w o X)
    // fragments of token block sb at xtr + 16 sb kXS * 2
    const uint32_t btr = (uint32_t)(((4 * q4 + j16 / 4) * NS + 4 * (j16 % 4)) * 2);
    const uint32_t xtr = (uint32_t)(((4 * q4 + j16 / 4) * kXS + p0 + 4 * (j16 % 4)) * 2);
    const unsigned char* sBb = reinterpret_cast<const unsigned char*>(sB);
    const unsigned char* sXb = reinterpret_cast<const unsigned char*>(sX);
    auto xfrag = [&](int sb) {
        const uint32_t o = xtr + (uint32_t)(16 * sb * kXS * 2);
        return Split4{tr_read(sXb, o), tr_read(sXb, o + cX * 2)};
    };

    const int nchunks = (tend - tbeg + Q - 1) / Q;
    CR regs;
    if (nchunks > 0) {
        load_bc(tbeg, regs);
        load_xz(tbeg, regs);
    }

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = tbeg + c * Q;
        const bool tail = t0 + Q > tend;              // chunk-uniform
        const bool tok_ok = t0 + lane < tend;
        // ---- segmented cumulative sum of dt*A (log2 domain), lane = token; every
        // wave of a head computes it (no wave waits for another)
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

        // this chunk's x and z stay in registers until the last use; the next
        // chunk's are loaded after it (load_xz), its B, C, dt earlier (load_bc)
        float4* xv = regs.x;
        const float4* zv = regs.z;
        if (tail) {
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
                if (t0 + 16 * ti + j16 >= tend) xv[ti] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        lds_barrier();     // the previous chunk's LDS readers are done

        // chunk-state weight of token `lane`: decay to the chunk end, last segment only
        sWw[lane] = lane >= wseg ? fast_exp2(cs_end - cs) * dtl : 0.0f;
        // ---- stage B (and C) row-major; rows past the end are zero
#pragma unroll
        for (int it = 0; it < CR::NIT; ++it) {
            const int item = tid + it * NTH;
            if (item < CR::NITEMS) {
                const int rp = item / CR::CPR, col = item % CR::CPR;
                const int s = 2 * rp, n0 = col * 4;
                uint4 b0 = regs.b[it][0], b1 = regs.b[it][1];
                uint4 c0 = regs.c[it][0], c1 = regs.c[it][1];
                if (tail) {
                    const uint4 zz = make_uint4(0, 0, 0, 0);
                    if (t0 + s >= tend) { b0 = zz; c0 = zz; }
                    if (t0 + s + 1 >= tend) { b1 = zz; c1 = zz; }
                }
                const float* fb0 = reinterpret_cast<const float*>(&b0);
                const float* fb1 = reinterpret_cast<const float*>(&b1);
                pst4(sB, cB, s * NS + n0, fb0[0], fb0[1], fb0[2], fb0[3]);
                pst4(sB, cB, (s + 1) * NS + n0, fb1[0], fb1[1], fb1[2], fb1[3]);
                if (FULL) {
                    const float* fc0 = reinterpret_cast<const float*>(&c0);
                    const float* fc1 = reinterpret_cast<const float*>(&c1);
                    pst4(sC, cB, s * NS + n0, fc0[0], fc0[1], fc0[2], fc0[3]);
                    pst4(sC, cB, (s + 1) * NS + n0, fc1[0], fc1[1], fc1[2], fc1[3]);
                }
            }
        }
        // ---- this wave's columns of X (kFull) or of w o X (kStateOnly), row-major
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int t = 16 * ti + j16;
            const float w = FULL ? 1.0f : sWw[t];
            pst4(sX, cX, t * kXS + p0 + 4 * q4, w * xv[ti].x, w * xv[ti].y, w * xv[ti].z, w * xv[ti].w);
        }
        // ---- per-token scalars of the chunk, once per head
        if (FULL && (wave & 3) == 0) {
            sCs[lane] = cs;
            sDt[lane] = dtl;
            sSeg[lane] = seg < 0 ? 0 : seg;
            // Yoff applies while no document has started in [chunk start, t]
            sEo[lane] = seg < 0 ? fast_exp2(cs) : 0.0f;
        }
        lds_barrier();     // staged tiles and scalars are visible
        if (c + 1 < nchunks) {
            load_bc(t0 + Q, regs);
            if (!FULL) load_xz(t0 + Q, regs);
        }
        // kFull: the first token tile whose rows need output (rows before
        // y_row0 need none), and whether this chunk's state is still needed:
        // by a later chunk, or as the final state
        const int T0 = FULL ? min(max(a.y_row0 - t0, 0), Q) / 16 : 0;
        const bool need_state = !FULL || c + 1 < nchunks || (a.final_state && k == a.K - 1);

        if (FULL) {
            // ---- G^T tiles (this wave's share of the lower triangle), each turned
            // into every head's M^T tile
            for (int kt = wave; kt < kNumMTiles; kt += NW) {
                int si, ti;
                mtile(kt, si, ti);
                if (ti < T0) continue;                    // feeds only rows that need no output
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nb = 0; nb < NT; nb += 2) {
                    const Split4 a0 = pld(sB, cB, (16 * si + j16) * NS + 16 * nb + 4 * q4);
                    const Split4 b0 = pld(sC, cB, (16 * ti + j16) * NS + 16 * nb + 4 * q4);
                    const Split4 a1 = nb + 1 < NT ? pld(sB, cB, (16 * si + j16) * NS + 16 * (nb + 1) + 4 * q4)
                                                  : split_zero();
                    const Split4 b1 = nb + 1 < NT ? pld(sC, cB, (16 * ti + j16) * NS + 16 * (nb + 1) + 4 * q4)
                                                  : split_zero();
                    acc = mma_split(acc, a0, a1, b0, b1);
                }
                // acc[r] = G^T[s = 16si + 4q4 + r][t = 16ti + j16]
                const int t = 16 * ti + j16;
                bool ok[4];
                for (int e = 0; e < HPW; ++e) {
                    const float* sce = sScal + 4 * Q * e;
                    const float cst = sce[t];
                    const int segt = reinterpret_cast<const int*>(sce + 2 * Q)[t];
                    const float4 css = *reinterpret_cast<const float4*>(sce + 16 * si + 4 * q4);
                    const float4 dts = *reinterpret_cast<const float4*>(sce + Q + 16 * si + 4 * q4);
                    f32x4 m;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = 16 * si + 4 * q4 + r;
                        ok[r] = (si < ti || s <= t) && (!has_bnd || s >= segt);
                        m[r] = ok[r] ? acc[r] * fast_exp2(cst - (&css.x)[r]) * (&dts.x)[r] : 0.0f;
                    }
                    pst4(plane(LD::oH + e * LD::HB + cX), cM, kt * 256 + lane * 4, m[0], m[1], m[2], m[3]);
                }
            }
            // split copy of the carried state for the C.H contraction
            Split4 hf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) hf[nt] = split4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
            lds_barrier();     // all M^T tiles are in LDS

            // ---- per token tile: Ydiag^T = X^T M^T, Yoff^T = H^T C^T, then the output
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                if (ti < T0) continue;
                f32x4 yd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sb = 0; sb <= ti; sb += 2) {
                    const Split4 a0 = xfrag(sb);
                    const Split4 b0 = pld(sM, cM, mtile_index(sb, ti) * 256 + lane * 4);
                    const bool two = sb + 1 <= ti;
                    const Split4 a1 = two ? xfrag(sb + 1) : split_zero();
                    const Split4 b1 = two ? pld(sM, cM, mtile_index(sb + 1, ti) * 256 + lane * 4) : split_zero();
                    yd = mma_split(yd, a0, a1, b0, b1);
                }
                f32x4 yo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nb = 0; nb < NT; nb += 2) {
                    const Split4 c0 = pld(sC, cB, (16 * ti + j16) * NS + 16 * nb + 4 * q4);
                    const Split4 c1 = nb + 1 < NT ? pld(sC, cB, (16 * ti + j16) * NS + 16 * (nb + 1) + 4 * q4)
                                                  : split_zero();
                    const Split4 h1 = nb + 1 < NT ? hf[nb + 1] : split_zero();
                    yo = mma_split(yo, hf[nb], h1, c0, c1);
                }
                // lane holds y[t = 16ti + j16][p = p0 + 4q4 + r]
                const int t = 16 * ti + j16;
                const float eo = sEo[t];
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = fmaf(Dh, (&xv[ti].x)[r], fmaf(eo, yo[r], yd[r]));
                if (gate) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] *= silu_f((&zv[ti].x)[r]);
                }
                if (!tail || t0 + t < tend)
                    *reinterpret_cast<float4*>(reinterpret_cast<char*>(yg + (size_t)t0 * a.y_stride) +
                                               row_bytes(t, (int)a.y_stride, 0, 4)) = make_float4(o[0], o[1], o[2], o[3]);
            }
            // ---- w o X over this wave's own X columns (only this wave reads them,
            // and its LDS operations are performed in order)
            if (need_state) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const int t = 16 * ti + j16;
                    const float w = sWw[t];
                    pst4(sX, cX, t * kXS + p0 + 4 * q4, w * xv[ti].x, w * xv[ti].y, w * xv[ti].z, w * xv[ti].w);
                }
            }
            if (c + 1 < nchunks) load_xz(t0 + Q, regs);
        }
        if (!need_state) continue;   // the last chunk, no final state wanted: its state goes nowhere

        // ---- chunk state S = B^T (w o X): lane holds S[n = 16nt + 4q4 + r][p0 + j16],
        // then the state passing, strictly in chunk order.  B^T comes from the
        // row-major B planes through transposed reads.  A chunk holding a
        // document start drops the carried state: decay 0 (a multiply by
        // exactly zero of a finite state, so the result is S).
        const float dec = has_bnd ? 0.0f : fast_exp2(cs_end);
        // this wave's (w o X)^T fragments are the same for every n tile
        Split4 xwf[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) xwf[sb] = xfrag(sb);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; sb += 2) {
                const uint32_t o0 = btr + (uint32_t)((16 * sb * NS + 16 * nt) * 2);
                const uint32_t o1 = btr + (uint32_t)((16 * (sb + 1) * NS + 16 * nt) * 2);
                const Split4 a0 = {tr_read(sBb, o0), tr_read(sBb, o0 + cB * 2)};
                const Split4 a1 = {tr_read(sBb, o1), tr_read(sBb, o1 + cB * 2)};
                acc = mma_split(acc, a0, a1, xwf[sb], xwf[sb + 1]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Hs[nt][r] = fmaf(dec, Hs[nt][r], acc[r]);
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
        if (lane == 0 && (wave & 3) == 0) a.dec[u] = reset ? -1.0f : fast_exp2(log2dec);
        if (k == 0 && a.h0) {
            // the main pass reads this copy instead of init_state
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<float4*>(a.h0 + st_off + 16 * nt) =
                    *reinterpret_cast<const float4*>(a.init_state + st_off + 16 * nt);
        }
    }
}

// ============================================================================
// bf16 kernel: every per-chunk input is staged by LDS DMA.
//
// A workgroup owns HPW heads that share one B/C group (4 waves per head; wave
// w -> head w / 4, channels 16 (w mod 4) .. +16) and one superchunk of one
// batch row.  B, C and the heads' X rows of a chunk stream from HBM straight
// into row-major LDS tiles with global_load_lds (16 bytes per lane, lane-
// linear destination) one chunk ahead of the compute, into the other of two
// stages.  B and C are staged once for the HPW heads and each G^T tile
// (B C^T) is built once and turned into every head's M^T tile.  Transposed
// operands (B^T for the chunk state, X^T and (w o X)^T) come from the same
// row-major tiles through ds_read_b64_tr_b16: in each 16-lane group, result
// lane j element e is element (j mod 4) of source lane 4e + j/4, so a lane
// (q, m) that addresses row 4q + m/4, column 4(m mod 4) of a tile receives
// column m, rows 4q..4q+3 -- the operand fragment of the transposed tile.
// z (per wave: its 16 channels) and, for the head's lead wave, dt and the
// document ids also arrive by DMA, into wave-private buffers refilled right
// after they are read.
//
// Nothing in the chunk loop is an ordinary global load, so the compiler has
// no reason to wait on the vector-memory counter there; the waits are explicit
// and rely on one wave's vector-memory operations completing in issue order.
// Per chunk c a wave issues, in this order:
//   [lead: dt, doc ids of c+1] -- barrier A -- [B, C, X copies of c+1]
//   -- barrier B -- [4 y stores of c] [2 z copies of c+1]
// so at the top of chunk c+1 "its B/C/X (and dt/doc) have landed" is "at most
// 6 newer operations are outstanding", and z of chunk c is in once at most
// (this wave's B/C/X copies of c+1) remain.  y goes out through buffer stores
// whose range check drops rows past the unit's end, so every chunk issues
// exactly 4.  Barriers wait only for LDS traffic (lgkmcnt), never for the
// copies in flight.
// ============================================================================
// LDS DMA: lane l's 16 (or 4) bytes at base + voff land at lds + 16 l (4 l).
// base and lds are wave-uniform.  Written as inline assembly so the compiler
// does not model the copy: it would otherwise wait for every copy in flight
// before any LDS read it cannot prove disjoint.  M0 (the LDS destination) is
// saved and restored inside the statement; one wait state separates its write
// from the copy.
// The LDS address of a generic pointer into LDS is its low 32 bits (the LDS
// aperture is 4 GiB aligned); an address-space cast would add null checks of
// both pointer forms to every copy.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const unsigned char* lds) {
    uint32_t m0_saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved)
        : "v"(voff), "s"(uniform_ptr(base)), "s"(lds_addr(lds))
        : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, const unsigned char* lds) {
    uint32_t m0_saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved)
        : "v"(voff), "s"(uniform_ptr(base)), "s"(lds_addr(lds))
        : "memory");
}
// At most n of this wave's vector-memory operations still outstanding.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
// The same for a wave-uniform n in [0, 63] (larger n waits for 63): a chain of
// scalar compares picks the immediate.
template <int LO = 0>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
    if constexpr (LO == 63) {
        wait_vmcnt<63>();
    } else {
        if (n <= LO) wait_vmcnt<LO>();
        else wait_vmcnt_n<LO + 1>(n);
    }
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

// ---------------------------------------------------------------------------
// Fused conv prologue (CV kernels): a chunk's raw B (and C) and X tiles are
// convolved (k = 4) and activated in place in LDS before any contraction reads
// them.  A lane owns one 4-byte word (two channels) of the tile rows; waves
// are grouped WPS to a row segment of R consecutive rows, which the lane walks
// in order with the three previous raw rows in registers.  The arithmetic (the
// fp32 fma chain bias + w0 x(t-3) + w1 x(t-2) + w2 x(t-1) + w3 x(t), SiLU,
// rounding to bf16) and the document handling (history zeroed where a
// document starts, halo rows cut at starts inside them) are those of
// ssd_conv_fwd, so the contractions see bit-identical operands.
template <int N, int HPW, bool WITH_C, int NW>
struct ConvMap {
    static constexpr int NWB = (WITH_C ? 2 : 1) * (N / 2);   // B (and C) words per row
    static constexpr int WD = NWB + 32 * HPW;                 // words per row, X last
    static constexpr int WPS = (WD + 63) / 64;                // waves per row segment
    static constexpr int RS = NW / WPS;                       // row segments
    static constexpr int R = (Q + RS - 1) / RS;               // rows per segment
};

// One lane's conv word inside a stage, swizzled like the copies: row r of the
// word's tile sits at (tp + r * rb) ^ (f(r) << 4), f(r) = (r >> rl_sh) & cpr_m
// (tp = tile offset | 16-byte piece << 4 | byte in the piece; the tile offset
// is a multiple of rb, so the xor only touches the piece bits).
struct ConvWord {
    uint32_t tp;
    int rb, rl_sh, cpr_m;
};
__device__ __forceinline__ ConvWord conv_word(uint32_t tile, int rb, int wb) {
    const int rl = rb >= 256 ? 1 : 256 / rb;
    return {tile | (uint32_t)((wb >> 2) << 4) | (uint32_t)((wb & 3) * 4), rb,
            rl == 1 ? 0 : (rl == 2 ? 1 : (rl == 4 ? 2 : 3)), rb / 16 - 1};
}
// RBU > 0: every lane's tile rows are RBU bytes, so the swizzle is wave-uniform
// and only tp is per lane.
template <int RBU>
__device__ __forceinline__ uint32_t conv_off(const ConvWord& w, int r) {
    if constexpr (RBU > 0) {
        constexpr int rl = RBU >= 256 ? 1 : 256 / RBU;
        constexpr int sh = rl == 1 ? 0 : (rl == 2 ? 1 : (rl == 4 ? 2 : 3));
        return (w.tp + (uint32_t)(r * RBU)) ^ ((uint32_t)((r >> sh) & (RBU / 16 - 1)) << 4);
    } else {
        return (w.tp + (uint32_t)(r * w.rb)) ^ ((uint32_t)((r >> w.rl_sh) & w.cpr_m) << 4);
    }
}
// The in-place conv of one lane's word over rows [r0, r1) of a stage.  v3,
// v2, v1: the raw words of rows r0-3 .. r0-1, already cut at document
// starts before r0; smask bit r: row r starts a document (the history is
// zeroed before it).  Rows are independent given the raw history, so whole
// groups of four are read ahead of their arithmetic, with no per-row bound
// test; the last r1 - r0 mod 4 rows go one at a time.  DOCS: some row of
// [r0, r1) starts a document (else the per-row test is left out); SILU: the
// activation (else the identity).
template <int RBU, bool DOCS, bool SILU>
__device__ __forceinline__ void conv_rows_t(unsigned char* stg, const ConvWord& cw, int r0, int r1, uint64_t smask,
                                            uint32_t v3, uint32_t v2, uint32_t v1, const float (&w)[2][4],
                                            const float (&cb)[2]) {
    float h3[2] = {bf16_lo(v3), bf16_hi(v3)}, h2[2] = {bf16_lo(v2), bf16_hi(v2)},
          h1[2] = {bf16_lo(v1), bf16_hi(v1)};
    auto row = [&](int r, uint32_t cur) __attribute__((always_inline)) {
        if (DOCS && ((smask >> r) & 1)) {
            h3[0] = h3[1] = h2[0] = h2[1] = h1[0] = h1[1] = 0.0f;
        }
        const float c[2] = {bf16_lo(cur), bf16_hi(cur)};
        float o[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float v = cb[e];
            v = fmaf(w[e][0], h3[e], v);
            v = fmaf(w[e][1], h2[e], v);
            v = fmaf(w[e][2], h1[e], v);
            v = fmaf(w[e][3], c[e], v);
            o[e] = SILU ? silu_f(v) : v;
            h3[e] = h2[e];
            h2[e] = h1[e];
            h1[e] = c[e];
        }
        *reinterpret_cast<uint32_t*>(stg + conv_off<RBU>(cw, r)) = pack_bf16x2(o[0], o[1]);
    };
    int r = r0;
#pragma unroll 1
    for (; r + 4 <= r1; r += 4) {
        uint32_t cur[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) cur[u] = *reinterpret_cast<const uint32_t*>(stg + conv_off<RBU>(cw, r + u));
#pragma unroll
        for (int u = 0; u < 4; ++u) row(r + u, cur[u]);
    }
#pragma unroll 1
    for (; r < r1; ++r) row(r, *reinterpret_cast<const uint32_t*>(stg + conv_off<RBU>(cw, r)));
}
// The row loop specialised on the (wave-uniform) document starts among its
// rows and the activation, so neither costs a select per row.
template <int RBU>
__device__ __forceinline__ void conv_rows(unsigned char* stg, const ConvWord& cw, int r0, int r1, uint64_t smask,
                                          uint32_t v3, uint32_t v2, uint32_t v1, const float (&w)[2][4],
                                          const float (&cb)[2], bool silu) {
    const int n = r1 - r0;
    const uint64_t rows = n >= 64 ? ~0ull : ((1ull << n) - 1) << r0;
    if (smask & rows) {
        if (silu) conv_rows_t<RBU, true, true>(stg, cw, r0, r1, smask, v3, v2, v1, w, cb);
        else conv_rows_t<RBU, true, false>(stg, cw, r0, r1, smask, v3, v2, v1, w, cb);
    } else {
        if (silu) conv_rows_t<RBU, false, true>(stg, cw, r0, r1, smask, v3, v2, v1, w, cb);
        else conv_rows_t<RBU, false, false>(stg, cw, r0, r1, smask, v3, v2, v1, w, cb);
    }
}

// LDS plan of the full pass: NS stages of a chunk's inputs -- B, C and the
// heads' X tiles, the heads' dt / doc ids and (ZR) every wave's z tile --
// then the heads' M^T fragments, (!ZR) one z tile per wave, and two buffers
// of per-token scalars.  A chunk's tiles are copied NS - 1 chunks ahead of
// its compute; z in the ring likewise, z outside it (NS = 2 only) right after
// the previous chunk's outputs.  MS: M^T is held as bf16 high and low halves,
// else as one bf16 rounding.
template <int N, int HPW, int NS_ = 2, bool ZR_ = true, bool MS_ = true>
struct LdsBf {
    static constexpr int NS = NS_;
    static constexpr bool ZR = ZR_, MS = MS_;
    static constexpr int NW = 4 * HPW;                // waves
    static constexpr int RB = N * 2;                  // bytes per B / C row
    static constexpr int XB = 128;                    // bytes per X row of one head (64 channels)
    static constexpr int TB = Q * RB;                 // B or C tile
    static constexpr int TX = Q * XB;                 // X tile of one head
    static constexpr int ZW = Q * 32;                 // one wave's z tile [Q][16] bf16
    static constexpr int DB = HPW * 3 * Q * 4;        // per head: dt, doc, doc of the previous token [Q] each
    static constexpr int oB = 0, oC = TB, oX = 2 * TB;   // then the HPW X tiles
    static constexpr int oZs = oX + HPW * TX;         // the waves' z tiles (ZR)
    static constexpr int oDs = oZs + (ZR ? NW * ZW : 0);   // the heads' dt / doc ids (ZR)
    static constexpr int STAGE = oDs + (ZR ? DB : 0);
    // one head's M^T tiles as bf16 fragments: the high halves of the 10 tiles,
    // then (MS) the low halves (M = hi + lo to 2^-16 relative)
    static constexpr int MB = (MS ? 2 : 1) * kNumMTiles * 512;
    static constexpr int oM = NS * STAGE;
    static constexpr int oZ1 = oM + HPW * MB;         // the waves' z tiles (!ZR)
    static constexpr int oD1 = oZ1 + (ZR ? 0 : NW * ZW);   // the heads' dt / doc ids (!ZR)
    static constexpr int oS = oD1 + (ZR ? 0 : DB);
    // per-token scalars of one chunk, floats: per head cs, dt, eo, w [Q] each;
    // then the segment start per token [Q] (int); cs_end per head; last_seg
    static constexpr int SC_SEG = 4 * HPW * Q;
    static constexpr int SC_END = SC_SEG + Q;
    static constexpr int SC_LAST = SC_END + HPW;
    // fused conv: document starts of the chunk (64-bit mask), and of the two
    // tokens before it (bit 0: t0 - 1, bit 1: t0 - 2)
    static constexpr int SC_ST = SC_LAST + 1;
    static constexpr int SCW = (SC_ST + 3 + 3) / 4 * 4;
    static constexpr int bytes = oS + 2 * SCW * 4;
    // 16-byte copies per chunk: rows per instruction of a B/C tile and of an X tile
    static constexpr int RPI_B = 64 / (RB / 16);
    static constexpr int NI_B = Q / RPI_B;
    static constexpr int NI_X = Q / 8;
    static constexpr int NI_BC = 2 * NI_B;
    static constexpr int NI = NI_BC + HPW * NI_X;
    static constexpr int NI_W = (NI + NW - 1) / NW;   // most copies a wave issues
    static constexpr int NI_MIN = NI / NW;            // fewest
};

template <int N, bool SP, int HPW, bool CV, int NS, bool ZR, bool MS>
__global__ __launch_bounds__(256 * HPW) void ssd_scan_bf16_kernel(ScanArgs a) {
    using LD = LdsBf<N, HPW, NS, ZR, MS>;
    static_assert(LD::bytes <= 163840, "LDS plan exceeds a CU");
    static_assert(ZR || NS == 2, "z outside the ring is single-buffered");
    static_assert(SP || !CV, "the fused conv takes raw dt through the softplus");
    constexpr int NT = N / 16;
    constexpr int NW = LD::NW;
    constexpr int RB = LD::RB, XB = LD::XB;
    constexpr int CPR_B = RB / 16;
    using SB = Swz<RB>;
    using SX = Swz<XB>;

    extern __shared__ __align__(16) unsigned char smem[];
    float* scal = reinterpret_cast<float*>(smem + LD::oS);   // [2][SCW]

    const int L = a.L, H = a.H, G = a.G;
    const int HQ = H / HPW;
    const int KU = a.K;
    const int id = xcd_remap(blockIdx.x, a.B * HQ * KU);
    const int hq = id % HQ;
    const int k = (id / HQ) % KU;
    const int b = id / (HQ * KU);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hh = wave >> 2;                  // head of this wave within the workgroup
    const int h = hq * HPW + hh;
    const int g = (hq * HPW) / (H / G);
    // Lead waves: wave e < HPW computes the per-token scalars of head e.  They
    // are the first wave of each SIMD, which the SIMD's issue arbitration
    // favours, so the scalar work starts as soon as the chunk's inputs land.
    const bool lead = wave < HPW;
    const int lh = lead ? wave : hh;           // the head whose scalars a lead wave computes
    const int h_l = hq * HPW + lh;
    const int q4 = lane >> 4;
    const int j16 = lane & 15;
    const int p0 = (wave & 3) * 16;
    const float A2l = a.A[h_l] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float dtbl = (a.dt_softplus && a.dt_bias) ? a.dt_bias[h_l] : 0.0f;
    const int tbeg = k * a.S;
    const int tend = min(tbeg + a.S, L);
    const int tl = tend - 1;
    const bool gate = a.z != nullptr;
    const bool docs = a.doc != nullptr;

    // ---- global bases (uniform)
    const uint16_t* xhead = static_cast<const uint16_t*>(a.x) + (size_t)b * a.Lb * a.x_stride + (size_t)hq * HPW * 64;
    const uint16_t* zbase = gate ? static_cast<const uint16_t*>(a.z) + (size_t)b * a.Lb * a.z_stride + (size_t)h * 64 + p0
                                 : xhead + hh * 64 + p0;   // stand-in rows keep the operation count fixed
    const int Zs2 = (int)(gate ? a.z_stride : a.x_stride) * 2;
    const uint16_t* Bbase = static_cast<const uint16_t*>(a.Bm) + (size_t)b * a.Lb * a.B_stride + (size_t)g * N;
    const uint16_t* Cbase = static_cast<const uint16_t*>(a.Cm) + (size_t)b * a.Lb * a.C_stride + (size_t)g * N;
    // dt: fp32, or (CV) the raw bf16 dt, read as the 4-byte word holding heads h & ~1 and h | 1
    const void* dtbase = CV ? static_cast<const void*>(a.dt16 + (size_t)b * a.Lb * a.dt16_stride + (h_l & ~1))
                            : static_cast<const void*>(a.dt + (size_t)b * a.Lb * a.dt_stride + h_l);
    const int32_t* docbase = a.doc + (size_t)b * a.Lb;
    float* ybase = a.y + (size_t)b * a.Lb * a.y_stride + h * 64;
    const int Ds4 = CV ? (int)a.dt16_stride * 2 : (int)a.dt_stride * 4;
    const int Ys = (int)a.y_stride;

    // in stage st: this wave's z tile, and this head's dt, doc, doc-1
    auto zbuf = [&](int st) {
        return ZR ? smem + st * LD::STAGE + LD::oZs + wave * LD::ZW : smem + LD::oZ1 + wave * LD::ZW;
    };
    auto dbuf = [&](int st) {
        return (ZR ? smem + st * LD::STAGE + LD::oDs : smem + LD::oD1) + lh * 3 * Q * 4;
    };

    // Copy slots of this wave: slot j is copy instruction wave + NW j of the
    // chunk (B tile, then C tile, then the X tiles).  Per slot: the uniform
    // source base and row stride, the LDS destination, and the lane's tile row
    // and column byte offset (the swizzled piece this lane's 16 bytes land in).
    const char* s_base[LD::NI_W];
    int s_stride[LD::NI_W];        // bytes per row
    uint32_t s_lds[LD::NI_W];
    int s_row[LD::NI_W];
    uint32_t s_col[LD::NI_W];
    uint32_t s_off[LD::NI_W];      // the lane's byte offset in the chunk when no row is clamped
    bool s_on[LD::NI_W];
    constexpr bool kAllOn = LD::NI % NW == 0;   // every wave issues NI_W copies
#pragma unroll
    for (int j = 0; j < LD::NI_W; ++j) {
        const int i = wave + NW * j;
        s_on[j] = i < LD::NI;
        if (i < LD::NI_BC) {
            const bool isC = i >= LD::NI_B;
            const int ins = isC ? i - LD::NI_B : i;
            s_base[j] = reinterpret_cast<const char*>(isC ? Cbase : Bbase);
            s_stride[j] = (int)(isC ? a.C_stride : a.B_stride) * 2;
            s_lds[j] = (isC ? LD::oC : LD::oB) + ins * 1024;
            const int r = ins * LD::RPI_B + lane / CPR_B;
            s_row[j] = r;
            s_col[j] = (uint32_t)(((lane % CPR_B) ^ SB::f(r)) * 16);
        } else {
            const int ix = s_on[j] ? i - LD::NI_BC : 0;
            const int e = ix / LD::NI_X, ins = ix % LD::NI_X;
            s_base[j] = reinterpret_cast<const char*>(xhead + e * 64);
            s_stride[j] = (int)a.x_stride * 2;
            s_lds[j] = LD::oX + e * LD::TX + ins * 1024;
            const int r = ins * 8 + lane / (XB / 16);
            s_row[j] = r;
            s_col[j] = (uint32_t)(((lane % (XB / 16)) ^ SX::f(r)) * 16);
        }
        s_off[j] = (uint32_t)(s_row[j] * s_stride[j]) + s_col[j];
    }
    // vector-memory operations this wave issues per chunk for the tiles, and
    // (lead waves) for dt / doc ids: the exact counts its waits are built from
    const int n_tiles = (LD::NI - wave + NW - 1) / NW;
    const int n_scal = lead ? (docs ? 3 : 1) : 0;
    // B, C, X copies of the chunk at t0 into stage st; rows clamp to the unit's end
    // (slots j0 .. j1-1 of them)
    auto issue_tiles = [&](int t0, int st, int j0 = 0, int j1 = LD::NI_W) {
        const int lim = tl - t0;
        unsigned char* base = smem + st * LD::STAGE;
        if (lim >= Q - 1) {          // every row inside the unit: the precomputed offsets
#pragma unroll
            for (int j = 0; j < LD::NI_W; ++j)
                if (j >= j0 && j < j1 && (kAllOn || s_on[j]))
                    dma16(s_base[j] + (size_t)t0 * s_stride[j], s_off[j], base + s_lds[j]);
        } else {
#pragma unroll
            for (int j = 0; j < LD::NI_W; ++j)
                if (j >= j0 && j < j1 && (kAllOn || s_on[j]))
                    dma16(s_base[j] + (size_t)t0 * s_stride[j], (uint32_t)(min(s_row[j], lim) * s_stride[j]) + s_col[j],
                          base + s_lds[j]);
        }
    };
    // lead waves: dt and the doc ids of tokens t0 + lane and t0 + lane - 1
    auto issue_scalars = [&](int t0, int st) {
        const int rowl = min(lane, tl - t0);
        unsigned char* d = dbuf(st);
        dma4(static_cast<const char*>(dtbase) + (size_t)t0 * Ds4, (uint32_t)(rowl * Ds4), d);
        if (docs) {
            dma4(docbase, (uint32_t)(t0 + rowl) * 4, d + Q * 4);
            dma4(docbase, (uint32_t)max(t0 + rowl - 1, 0) * 4, d + 2 * Q * 4);
        }
    };
    // z of this wave's 16 channels: row r of the chunk -> zbuf + 32 r
    auto issue_z = [&](int t0, int st) {
        const int lim = tl - t0;
        const char* Zc = reinterpret_cast<const char*>(zbase + (size_t)t0 * (Zs2 / 2));
        unsigned char* zb = zbuf(st);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = min(32 * i + (lane >> 1), lim);
            dma16(Zc, (uint32_t)(row * Zs2) + (lane & 1) * 16, zb + i * 1024);
        }
    };
    // the chunk at t0 into stage st: n_grp operations of this wave (ZR: dt / doc
    // ids and z too; otherwise those follow their own schedule)
    const int n_grp = n_scal + n_tiles + 2;
    auto issue_chunk = [&](int t0, int st) {
        if constexpr (ZR) {
            if (lead) issue_scalars(t0, st);
            issue_tiles(t0, st);
            issue_z(t0, st);
        } else {
            issue_tiles(t0, st);
        }
    };
    // The same operations in two parts (part 0: dt / doc ids and the first half
    // of the tile copies; part 1: the rest and z), issued at two points of the
    // chunk loop: all waves issuing a chunk's copies at once would queue behind
    // one another in the CU's memory pipeline before their own compute.
    constexpr int kHalf = (LD::NI_W + 1) / 2;
    auto issue_chunk_part = [&](int t0, int st, int part) {
        if (part == 0) {
            if (ZR && lead) issue_scalars(t0, st);
            issue_tiles(t0, st, 0, kHalf);
        } else {
            issue_tiles(t0, st, kHalf, LD::NI_W);
            if constexpr (ZR) issue_z(t0, st);
        }
    };

    // the first chunks' copies go out before the state loads, so their latencies overlap
    const int nchunks = (tend - tbeg + Q - 1) / Q;
    if (!ZR && lead && nchunks > 0) issue_scalars(tbeg, 0);
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        if (j < nchunks) issue_chunk(tbeg + j * Q, j);
    if (!ZR && nchunks > 0) issue_z(tbeg, 0);

    // ---- initial state: the given one, then the superchunks before k folded in
    f32x4 Hs[NT];
    const size_t st_off = (((size_t)b * H + h) * 64 + p0 + j16) * N + 4 * q4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Hs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* h_init = a.K > 1 ? a.h0 : a.init_state;   // split: the pre-pass's copy
    if (h_init) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float4 v = *reinterpret_cast<const float4*>(h_init + st_off + 16 * nt);
            Hs[nt] = f32x4{v.x, v.y, v.z, v.w};
        }
    }
    // the preceding superchunks' local states, folded in order; their loads
    // are issued FOLD at a time so the fold costs ceil(k / FOLD) latencies
    constexpr int FOLD = 16 / NT < 4 ? 16 / NT : 4;
    for (int j0 = 0; j0 < k; j0 += FOLD) {
        float dj[FOLD];
        float4 v[FOLD][NT];
#pragma unroll
        for (int i = 0; i < FOLD; ++i) {
            const size_t u = ((size_t)b * H + h) * (a.K - 1) + min(j0 + i, k - 1);
            dj[i] = a.dec[u];
            const float* hl = a.hloc + u * 64 * N + (size_t)(p0 + j16) * N + 4 * q4;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) v[i][nt] = *reinterpret_cast<const float4*>(hl + 16 * nt);
        }
#pragma unroll
        for (int i = 0; i < FOLD; ++i) {
            if (j0 + i < k) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    Hs[nt][0] = dj[i] < 0.0f ? v[i][nt].x : fmaf(dj[i], Hs[nt][0], v[i][nt].x);
                    Hs[nt][1] = dj[i] < 0.0f ? v[i][nt].y : fmaf(dj[i], Hs[nt][1], v[i][nt].y);
                    Hs[nt][2] = dj[i] < 0.0f ? v[i][nt].z : fmaf(dj[i], Hs[nt][2], v[i][nt].z);
                    Hs[nt][3] = dj[i] < 0.0f ? v[i][nt].w : fmaf(dj[i], Hs[nt][3], v[i][nt].w);
                }
            }
        }
    }
    // settle the state loads here, before any copy is in flight
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(Hs[nt]));

    // ---- fused conv: this lane's word, its weights, and the raw halo rows of
    // the first chunk (the conv state at t = 0, else the three rows before)
    using CM = ConvMap<N, HPW, true, NW>;
    static_assert(!CV || (CM::RS >= 1 && CM::R >= 3 && (CM::RS - 1) * CM::R < Q), "conv row segments");
    const int cseg = wave / CM::WPS;
    const int cwi = (wave % CM::WPS) * 64 + lane;
    const bool c_on = CV && cseg < CM::RS && cwi < CM::WD;
    const int CD = H * 64 + 2 * G * N;              // conv_dim
    constexpr int RBU = RB == XB ? RB : 0;        // B/C and X rows alike: wave-uniform swizzle
    // the lane's word: its tile in a stage, its channel, its raw column in global memory
    auto conv_lane = [&](int wi, ConvWord& w, int& ch, const uint16_t*& src, int64_t& stride) {
        if (wi < N) {
            const bool isC = wi >= N / 2;
            const int wb = isC ? wi - N / 2 : wi;
            w = conv_word(isC ? LD::oC : LD::oB, RB, wb);
            ch = H * 64 + (isC ? G * N : 0) + g * N + 2 * wb;
            src = (isC ? Cbase : Bbase) + 2 * wb;
            stride = isC ? a.C_stride : a.B_stride;
        } else {
            const int e = (wi - N) / 32, wb = (wi - N) % 32;
            w = conv_word(LD::oX + e * LD::TX, XB, wb);
            ch = (hq * HPW + e) * 64 + 2 * wb;
            src = xhead + e * 64 + 2 * wb;
            stride = a.x_stride;
        }
    };
    ConvWord cw{};
    float cwt[2][4] = {}, cbias[2] = {};
    uint32_t hw3 = 0, hw2 = 0, hw1 = 0;            // raw rows t0-3, t0-2, t0-1 (segment 0)
    int pbits = 0;                                 // lead of head 0: starts at t0-1 (bit 0), t0-2 (bit 1)
    // the B/C columns of the conv state are written by the group's first workgroup
    const bool bc_owner = (hq * HPW) % (H / G) == 0;
    if constexpr (CV) {
        int ch;
        const uint16_t* src;
        int64_t cstride;
        conv_lane(min(cwi, CM::WD - 1), cw, ch, src, cstride);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float4 wv = *reinterpret_cast<const float4*>(a.conv_w + (size_t)(ch + e) * 4);
            cwt[e][0] = wv.x; cwt[e][1] = wv.y; cwt[e][2] = wv.z; cwt[e][3] = wv.w;
            cbias[e] = a.conv_b ? a.conv_b[ch + e] : 0.0f;
        }
        if (tbeg == 0) {
            if (a.cstate_in) {
                const uint16_t* si = static_cast<const uint16_t*>(a.cstate_in) + (size_t)b * 3 * CD + ch;
                hw3 = *reinterpret_cast<const uint32_t*>(si);
                hw2 = *reinterpret_cast<const uint32_t*>(si + CD);
                hw1 = *reinterpret_cast<const uint32_t*>(si + 2 * CD);
            }
        } else {   // tbeg >= 64
            hw3 = *reinterpret_cast<const uint32_t*>(src + (size_t)(tbeg - 3) * cstride);
            hw2 = *reinterpret_cast<const uint32_t*>(src + (size_t)(tbeg - 2) * cstride);
            hw1 = *reinterpret_cast<const uint32_t*>(src + (size_t)(tbeg - 1) * cstride);
            if (docs) {
                const int d1 = docbase[tbeg - 1], d2 = docbase[tbeg - 2], d3 = docbase[tbeg - 3];
                pbits = (d1 != d2 ? 1 : 0) | (d2 != d3 ? 2 : 0);
            }
        }
        pbits = __builtin_amdgcn_readfirstlane(pbits);
        // ---- conv state after the call: the raw rows L-3 .. L-1 (rows before 0
        // from the incoming conv state), cut at document starts inside them.
        // Inputs only, so the last superchunk writes it up front (the caller's
        // conv state buffers do not overlap).
        const bool own = cwi < N ? bc_owner : true;
        if (a.cstate_out && k == a.K - 1 && c_on && cseg == 0 && own) {
            uint32_t sv[3];
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int u = L - 3 + i;
                if (u >= 0) {
                    sv[i] = *reinterpret_cast<const uint32_t*>(src + (size_t)u * cstride);
                } else {
                    sv[i] = a.cstate_in ? *reinterpret_cast<const uint32_t*>(
                                              static_cast<const uint16_t*>(a.cstate_in) + (size_t)b * 3 * CD +
                                              (size_t)(3 + u) * CD + ch)
                                        : 0u;
                }
            }
            if (docs) {
                if (L >= 3 && docbase[L - 2] != docbase[L - 3]) sv[0] = 0;            // a start at L-2
                if (L >= 2 && docbase[L - 1] != docbase[L - 2]) sv[0] = sv[1] = 0;    // a start at L-1
            }
            uint16_t* so = static_cast<uint16_t*>(a.cstate_out) + (size_t)b * 3 * CD + ch;
#pragma unroll
            for (int i = 0; i < 3; ++i) *reinterpret_cast<uint32_t*>(so + (size_t)i * CD) = sv[i];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            asm volatile("" : "+v"(cbias[e]));
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(cwt[e][j]));
        }
        asm volatile("" : "+v"(hw3), "+v"(hw2), "+v"(hw1));
    }


    for (int c = 0; c < nchunks; ++c) {
        const int t0 = tbeg + c * Q;
        const int st = c % NS;
        const bool more = c + 1 < nchunks;
        const unsigned char* sB = smem + st * LD::STAGE + LD::oB;
        const unsigned char* sC = smem + st * LD::STAGE + LD::oC;
        const unsigned char* sX = smem + st * LD::STAGE + LD::oX + hh * LD::TX;
        float* sc = scal + (c & 1) * LD::SCW;      // this chunk's scalars
        float* sch = sc + hh * 4 * Q;              // ... of this wave's head: cs, dt, eo, w

        // every input of chunk c has landed (z outside the ring: every other
        // input).  Newer operations of this wave: the 4 y stores of each of the
        // last min(c, NS-1) chunks, the copies of the chunks after c already
        // issued (at most NS-2 of them), and (!ZR) the z copies of chunk c.
        if constexpr (!ZR) {
            if (c == 0) wait_vmcnt<2>();
            else wait_vmcnt<6>();
        } else if constexpr (NS == 2) {
            if (c == 0) wait_vmcnt<0>();
            else wait_vmcnt<4>();
        } else {
            wait_vmcnt_n(4 * min(c, NS - 1) + n_grp * max(0, min(NS - 2, nchunks - 1 - c)));
        }
        // ---- lead waves: segmented cumulative sum of dt*A (log2 domain), lane = token
        if (lead) {
            const bool tok_ok = t0 + lane < tend;
            const unsigned char* db = dbuf(st);
            float dtl = reinterpret_cast<const float*>(db)[lane];
            const int d0 = reinterpret_cast<const int*>(db)[Q + lane];
            const int d1 = reinterpret_cast<const int*>(db)[2 * Q + lane];
            lds_wait();
            if (!ZR && more) issue_scalars(t0 + Q, 0);     // refilled right after it is read
            if (CV) {
                const uint32_t wd = __float_as_uint(dtl);
                dtl = (h_l & 1) ? bf16_hi(wd) : bf16_lo(wd);
            }
            if (SP) dtl = softplus_f(dtl + dtbl);
            if (!tok_ok) dtl = 0.0f;
            const int bnd = (docs && tok_ok && t0 + lane > 0 && d0 != d1) ? 1 : 0;
            if (CV) {
                const uint64_t m = __ballot(bnd);
                if (lh == 0 && lane == 0) {
                    int* sci = reinterpret_cast<int*>(sc);
                    sci[LD::SC_ST] = (int)(uint32_t)m;
                    sci[LD::SC_ST + 1] = (int)(uint32_t)(m >> 32);
                    sci[LD::SC_ST + 2] = pbits;
                }
                pbits = (int)(m >> 63) | (int)((m >> 61) & 2);   // for the next chunk
            }
            float cs = dtl * A2l;
            int seg = bnd ? lane : -1;
            wave_segscan(cs, bnd, seg);
            const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
            const int last_seg = __builtin_amdgcn_readlane(seg, 63);
            const int wseg = last_seg >= 0 ? last_seg : 0;
            float* schl = sc + lh * 4 * Q;         // head lh's cs, dt, eo, w
            schl[lane] = cs;
            schl[Q + lane] = dtl;
            schl[2 * Q + lane] = seg < 0 ? fast_exp2(cs) : 0.0f;
            schl[3 * Q + lane] = lane >= wseg ? fast_exp2(cs_end - cs) * dtl : 0.0f;
            if (lh == 0) reinterpret_cast<int*>(sc)[LD::SC_SEG + lane] = seg < 0 ? 0 : seg;
            if (lane == 0) {
                sc[LD::SC_END + lh] = cs_end;
                if (lh == 0) reinterpret_cast<int*>(sc)[LD::SC_LAST] = last_seg;
            }
        }
        lds_barrier();                   // A: chunk c tiles + scalars visible; chunk c-1 readers done
        // refill the stage chunk c-1 used with chunk c + NS - 1: part 0 now, part 1
        // after this wave's first G^T product (or its tile loop)
        const bool refill = c + NS - 1 < nchunks;
        bool refill1 = refill;
        if (refill) issue_chunk_part(t0 + (NS - 1) * Q, (c + NS - 1) % NS, 0);
        const float cs_end = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sc[LD::SC_END + hh])));
        const int last_seg = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(sc)[LD::SC_LAST]);
        const bool has_bnd = last_seg >= 0;

        if constexpr (CV) {
            // ---- conv + activation of the chunk's raw B, C and X tiles, in place
            unsigned char* stg = smem + st * LD::STAGE;
            const int* sci = reinterpret_cast<const int*>(sc);
            const uint64_t smask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(sci[LD::SC_ST + 1]) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane(sci[LD::SC_ST]);
            const int r0 = cseg * CM::R;
            auto ldw = [&](int r) { return *reinterpret_cast<const uint32_t*>(stg + conv_off<RBU>(cw, r)); };
            uint32_t v3 = 0, v2 = 0, v1 = 0;
            int pb = 0;
            if (c_on) {
                if (cseg == 0) {
                    v3 = hw3; v2 = hw2; v1 = hw1;
                    pb = __builtin_amdgcn_readfirstlane(sci[LD::SC_ST + 2]);
                    if (more) { hw3 = ldw(Q - 3); hw2 = ldw(Q - 2); hw1 = ldw(Q - 1); }   // next chunk's halo
                } else {
                    v3 = ldw(r0 - 3); v2 = ldw(r0 - 2); v1 = ldw(r0 - 1);
                    pb = (int)((smask >> (r0 - 1)) & 1) | (int)(((smask >> (r0 - 2)) & 1) << 1);
                }
            }
            lds_barrier();               // C: every raw halo row is read before any row is overwritten
            if (c_on) {
                if (pb & 1) { v3 = 0; v2 = 0; }   // a document starts at r0 - 1
                if (pb & 2) v3 = 0;               // ... at r0 - 2
                conv_rows<RBU>(stg, cw, r0, min(r0 + CM::R, Q), smask, v3, v2, v1, cwt, cbias, a.act == 0);
            }
            lds_barrier();               // D: the convolved tiles are visible
        }

        {
            unsigned char* sM = smem + LD::oM;
            // ---- G^T = B C^T once per tile, then each head's decay and mask -> M^T fragments
            for (int kt = wave; kt < kNumMTiles; kt += NW) {
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
                if (refill1) {
                    issue_chunk_part(t0 + (NS - 1) * Q, (c + NS - 1) % NS, 1);
                    refill1 = false;
                }
                const int t = 16 * ti + j16;
                const int segt = reinterpret_cast<const int*>(sc)[LD::SC_SEG + t];
                bool ok[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * si + 4 * q4 + r;
                    ok[r] = (si < ti || s <= t) && (!has_bnd || s >= segt);
                }
#pragma unroll
                for (int e = 0; e < HPW; ++e) {
                    const float* sce = sc + e * 4 * Q;
                    const float cst = sce[t];
                    const float4 css = *reinterpret_cast<const float4*>(sce + 16 * si + 4 * q4);
                    const float4 dts = *reinterpret_cast<const float4*>(sce + Q + 16 * si + 4 * q4);
                    f32x4 m;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        m[r] = ok[r] ? acc[r] * fast_exp2(cst - (&css.x)[r]) * (&dts.x)[r] : 0.0f;
                    const FragBF mh = frag_from_f32(m);
                    *reinterpret_cast<FragBF*>(sM + e * LD::MB + kt * 512 + lane * 8) = mh;
                    if constexpr (MS) {
                        const f32x4 ml = {m[0] - bf16_lo(mh.a), m[1] - bf16_hi(mh.a), m[2] - bf16_lo(mh.b),
                                          m[3] - bf16_hi(mh.b)};
                        *reinterpret_cast<FragBF*>(sM + e * LD::MB + (kNumMTiles + kt) * 512 + lane * 8) =
                            frag_from_f32(ml);
                    }
                }
            }
            if (refill1) issue_chunk_part(t0 + (NS - 1) * Q, (c + NS - 1) % NS, 1);   // a wave without tiles
            FragBF hf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) hf[nt] = frag_from_f32(Hs[nt]);
            lds_barrier();   // B: all M^T tiles are in LDS
            if constexpr (!ZR) {
                // z of chunk c has landed: only this wave's copies of chunk c+1
                // (and, in lead waves, its dt / doc ids) may be newer
                if (more) wait_vmcnt_n(n_tiles + n_scal);
                else wait_vmcnt<0>();
            }

            // ---- per token tile: Ydiag^T = X^T M^T, Yoff^T = H^T C^T, output
            const unsigned char* sMh = sM + hh * LD::MB;
            const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                ybase + (size_t)t0 * a.y_stride, 0, (tend - t0) * Ys * 4, 0x00020000);
            // f of the transpose-read rows does not depend on the 16-row block sb
            const uint32_t xtr = SX::off(4 * q4 + j16 / 4, p0 + 4 * (j16 % 4));
            uint2 zr[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
                zr[ti] = *reinterpret_cast<const uint2*>(zbuf(st) + (16 * ti + j16) * 32 + q4 * 8);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 yd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sb = 0; sb <= ti; sb += 2) {
                    // X is exact in bf16; M^T enters as its high and (MS) low halves
                    const FragBF a0 = tr_read(sX, xtr + 16 * sb * XB);
                    const int m0 = mtile_index(sb, ti) * 512 + lane * 8;
                    const FragBF b0 = plain_read(sMh + m0);
                    // the tile pair (sb, ti), (sb+1, ti) is adjacent (mtile_index)
                    const bool two = sb + 1 <= ti;
                    const FragBF a1 = two ? tr_read(sX, xtr + 16 * (sb + 1) * XB) : FragBF{0u, 0u};
                    const FragBF b1 = two ? plain_read(sMh + m0 + 512) : FragBF{0u, 0u};
                    if constexpr (MS) {
                        const FragBF l0 = plain_read(sMh + kNumMTiles * 512 + m0);
                        const FragBF l1 = two ? plain_read(sMh + kNumMTiles * 512 + m0 + 512) : FragBF{0u, 0u};
                        yd = mma_bf16(yd, a0, a1, l0, l1);
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
                const float eo = sch[2 * Q + t];
                const uint2 xr = *reinterpret_cast<const uint2*>(sX + SX::off(t, p0 + 4 * q4));
                const float xs[4] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y)};
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = fmaf(Dh, xs[r], fmaf(eo, yo[r], yd[r]));
                // the gate factors silu(z) of the lane's 4 outputs
                if (gate) {
                    v[0] *= silu_f(bf16_lo(zr[ti].x));
                    v[1] *= silu_f(bf16_hi(zr[ti].x));
                    v[2] *= silu_f(bf16_lo(zr[ti].y));
                    v[3] *= silu_f(bf16_hi(zr[ti].y));
                }
                const u32x4_t o = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                   __float_as_uint(v[3])};
                // rows past the unit's end fall outside the buffer range and are dropped
                __builtin_amdgcn_raw_buffer_store_b128(o, yr, (uint32_t)(t * Ys + p0 + 4 * q4) * 4, 0, 0);
            }
            // every wave's output stores are issued before any wave goes on (and,
            // z outside the ring, refills its z tile): the four 64-byte pieces of
            // a y row (one per wave of the head) then reach the L2 close together,
            // which shortens the pass by ~8%
            lds_barrier();
            if constexpr (!ZR) {
                if (more) issue_z(t0 + Q, 0);
            }
        }

        // ---- chunk state S = B^T (w o X) from the row-major tiles via transpose reads
        FragBF xw[4];
        {
            const uint32_t xtr = SX::off(4 * q4 + j16 / 4, p0 + 4 * (j16 % 4));
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const FragBF xf = tr_read(sX, xtr + 16 * sb * XB);
                const float4 w = *reinterpret_cast<const float4*>(sch + 3 * Q + 16 * sb + 4 * q4);
                xw[sb].a = pack_bf16x2(w.x * bf16_lo(xf.a), w.y * bf16_hi(xf.a));
                xw[sb].b = pack_bf16x2(w.z * bf16_lo(xf.b), w.w * bf16_hi(xf.b));
            }
        }
        // a chunk holding a document start drops the carried state: decay 0
        // (a multiply by exactly zero of a finite state, so the result is S)
        const float dec = has_bnd ? 0.0f : fast_exp2(cs_end);
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
#pragma unroll
            for (int r = 0; r < 4; ++r) Hs[nt][r] = fmaf(dec, Hs[nt][r], acc[r]);
        }
    }

    if (a.final_state && k == a.K - 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<float4*>(a.final_state + st_off + 16 * nt) =
                make_float4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
    }

}

// ============================================================================
// bf16 state-only pre-pass of the sequence split.
//
// For superchunk k < K-1 of (b, head group) it runs the chunk-state recurrence
// from a zero state over the superchunk and stores the local end state (hloc)
// and the total decay (dec; negative if a document starts inside, i.e. the
// carried state is dropped there).  Only B, X, dt and the doc ids are read.
// A workgroup covers HPW heads of one B/C group with 4 / PB waves per head; a
// wave owns PB 16-channel blocks, so each B^T fragment it reads from LDS feeds
// PB MFMAs and the per-wave overheads (copy issue, waits) are shared by PB
// blocks.  Copies run NS - 1 chunks ahead through an NS-stage LDS ring; each
// stage also holds the chunk's dt and doc ids for the heads' lead waves.
// ============================================================================
template <int N, int HPW, int PB, int NS>
struct LdsPre {
    static constexpr int WPH = 4 / PB;                // waves per head
    static constexpr int NW = WPH * HPW;              // waves
    static constexpr int RB = N * 2, XB = 128;        // bytes per B row, per X row of one head
    static constexpr int TB = Q * RB, TX = Q * XB;
    static constexpr int oB = 0, oX = TB;             // B tile, then the HPW X tiles
    static constexpr int DB = HPW * 3 * Q * 4;        // per head: dt, doc, doc of the previous token [Q]
    static constexpr int oD = oX + HPW * TX;
    static constexpr int STAGE = oD + DB;
    static constexpr int oS = NS * STAGE;
    // scalars of one chunk (floats): per head w [Q]; cs_end per head; last_seg
    static constexpr int SC_END = HPW * Q;
    static constexpr int SC_LAST = SC_END + HPW;
    static constexpr int SC_ST = SC_LAST + 1;         // fused conv: document starts, as in LdsBf
    static constexpr int SCW = (SC_ST + 3 + 3) / 4 * 4;
    static constexpr int bytes = oS + 2 * SCW * 4;
    static constexpr int RPI_B = 64 / (RB / 16);      // B rows per 1 KiB copy
    static constexpr int NI_B = Q / RPI_B;
    static constexpr int NI_X = Q / 8;
    static constexpr int NI = NI_B + HPW * NI_X;      // copies per chunk
    static constexpr int NI_W = (NI + NW - 1) / NW;
};

template <int N, bool SP, int HPW, int PB, int NS, bool CV>
__global__ __launch_bounds__(64 * (4 / PB) * HPW) void ssd_scan_state_kernel(ScanArgs a) {
    using LD = LdsPre<N, HPW, PB, NS>;
    static_assert(LD::bytes <= 163840, "LDS plan exceeds a CU");
    static_assert(SP || !CV, "the fused conv takes raw dt through the softplus");
    constexpr int NT = N / 16;
    constexpr int NW = LD::NW, WPH = LD::WPH;
    constexpr int RB = LD::RB, XB = LD::XB;
    constexpr int CPR_B = RB / 16;
    using SB = Swz<RB>;
    using SX = Swz<XB>;

    extern __shared__ __align__(16) unsigned char smem[];
    float* scal = reinterpret_cast<float*>(smem + LD::oS);   // [2][SCW]

    const int L = a.L, H = a.H, G = a.G;
    const int HQ = H / HPW;
    const int KU = a.K - 1;
    const int id = xcd_remap(blockIdx.x, a.B * HQ * KU);
    const int hq = id % HQ;
    const int k = (id / HQ) % KU;
    const int b = id / (HQ * KU);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hh = wave / WPH;                 // head of this wave within the workgroup
    const int h = hq * HPW + hh;
    const int g = (hq * HPW) / (H / G);
    // Lead waves: wave e < HPW computes the per-token weights of head e (the
    // first wave of each SIMD, which its issue arbitration favours).
    const bool lead = wave < HPW;
    const int lh = lead ? wave : hh;           // the head whose weights a lead wave computes
    const int h_l = hq * HPW + lh;
    const int q4 = lane >> 4;
    const int j16 = lane & 15;
    const int p0 = (wave % WPH) * 16 * PB;     // first channel of this wave's blocks
    const float A2l = a.A[h_l] * kLog2e;
    const float dtbl = (a.dt_softplus && a.dt_bias) ? a.dt_bias[h_l] : 0.0f;
    const int tbeg = k * a.S;
    const int tend = min(tbeg + a.S, L);
    const int tl = tend - 1;
    const bool docs = a.doc != nullptr;

    const uint16_t* xhead = static_cast<const uint16_t*>(a.x) + (size_t)b * a.Lb * a.x_stride + (size_t)hq * HPW * 64;
    const uint16_t* Bbase = static_cast<const uint16_t*>(a.Bm) + (size_t)b * a.Lb * a.B_stride + (size_t)g * N;
    // dt: fp32, or (CV) the raw bf16 dt, read as the 4-byte word holding heads h & ~1 and h | 1
    const void* dtbase = CV ? static_cast<const void*>(a.dt16 + (size_t)b * a.Lb * a.dt16_stride + (h_l & ~1))
                            : static_cast<const void*>(a.dt + (size_t)b * a.Lb * a.dt_stride + h_l);
    const int32_t* docbase = a.doc + (size_t)b * a.Lb;
    const int Ds4 = CV ? (int)a.dt16_stride * 2 : (int)a.dt_stride * 4;

    // copy slots of this wave: copy wave + NW j of the chunk (B tile, then X tiles)
    const char* s_base[LD::NI_W];
    int s_stride[LD::NI_W];
    uint32_t s_lds[LD::NI_W];
    int s_row[LD::NI_W];
    uint32_t s_col[LD::NI_W];
    bool s_on[LD::NI_W];
    uint32_t s_off[LD::NI_W];   // the lane's offset when no row clamps
#pragma unroll
    for (int j = 0; j < LD::NI_W; ++j) {
        const int i = wave + NW * j;
        s_on[j] = i < LD::NI;
        if (i < LD::NI_B) {
            s_base[j] = reinterpret_cast<const char*>(Bbase);
            s_stride[j] = (int)a.B_stride * 2;
            s_lds[j] = LD::oB + i * 1024;
            const int r = i * LD::RPI_B + lane / CPR_B;
            s_row[j] = r;
            s_col[j] = (uint32_t)(((lane % CPR_B) ^ SB::f(r)) * 16);
        } else {
            const int ix = s_on[j] ? i - LD::NI_B : 0;
            const int e = ix / LD::NI_X, ins = ix % LD::NI_X;
            s_base[j] = reinterpret_cast<const char*>(xhead + e * 64);
            s_stride[j] = (int)a.x_stride * 2;
            s_lds[j] = LD::oX + e * LD::TX + ins * 1024;
            const int r = ins * 8 + lane / (XB / 16);
            s_row[j] = r;
            s_col[j] = (uint32_t)(((lane % (XB / 16)) ^ SX::f(r)) * 16);
        }
        s_off[j] = (uint32_t)(s_row[j] * s_stride[j]) + s_col[j];
    }
    const int n_tiles = (LD::NI - wave + NW - 1) / NW;
    const int n_scal = lead ? (docs ? 3 : 1) : 0;
    // (slots j0 .. j1-1 of them)
    auto issue_tiles = [&](int t0, int st, int j0, int j1) {
        const int lim = tl - t0;
        const bool whole = lim >= Q - 1;   // uniform: every row inside the unit
        unsigned char* base = smem + st * LD::STAGE;
#pragma unroll
        for (int j = 0; j < LD::NI_W; ++j) {
            if (j >= j0 && j < j1 && s_on[j]) {
                const char* src = s_base[j] + (size_t)t0 * s_stride[j];
                dma16(src, whole ? s_off[j] : (uint32_t)(min(s_row[j], lim) * s_stride[j]) + s_col[j],
                      base + s_lds[j]);
            }
        }
    };
    auto dbuf_of = [&](int st) -> unsigned char* { return smem + st * LD::STAGE + LD::oD + lh * 3 * Q * 4; };
    auto issue_scalars = [&](int t0, int st) {
        unsigned char* dbuf = dbuf_of(st);
        const int rowl = min(lane, tl - t0);
        dma4(static_cast<const char*>(dtbase) + (size_t)t0 * Ds4, (uint32_t)(rowl * Ds4), dbuf);
        if (docs) {
            dma4(docbase, (uint32_t)(t0 + rowl) * 4, dbuf + Q * 4);
            dma4(docbase, (uint32_t)max(t0 + rowl - 1, 0) * 4, dbuf + 2 * Q * 4);
        }
    };

    f32x4 Hs[PB][NT];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) Hs[pb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float log2dec = 0.0f;
    bool reset = false;

    // ---- fused conv: this lane's word (B or X), its weights, the first halo
    using CM = ConvMap<N, HPW, false, NW>;
    static_assert(!CV || (CM::RS >= 1 && CM::R >= 3 && (CM::RS - 1) * CM::R < Q), "conv row segments");
    const int cseg = wave / CM::WPS;
    const int cwi = (wave % CM::WPS) * 64 + lane;
    const bool c_on = CV && cseg < CM::RS && cwi < CM::WD;
    const int CD = H * 64 + 2 * G * N;              // conv_dim
    constexpr int RBU = RB == XB ? RB : 0;
    ConvWord cw{};
    float cwt[2][4] = {}, cbias[2] = {};
    uint32_t hw3 = 0, hw2 = 0, hw1 = 0;
    int pbits = 0;
    if constexpr (CV) {
        const int wi = min(cwi, CM::WD - 1);
        int ch;
        const uint16_t* src;
        int64_t cstride;
        if (wi < N / 2) {
            cw = conv_word(LD::oB, RB, wi);
            ch = H * 64 + g * N + 2 * wi;
            src = Bbase + 2 * wi;
            cstride = a.B_stride;
        } else {
            const int e = (wi - N / 2) / 32, wb = (wi - N / 2) % 32;
            cw = conv_word(LD::oX + e * LD::TX, XB, wb);
            ch = (hq * HPW + e) * 64 + 2 * wb;
            src = xhead + e * 64 + 2 * wb;
            cstride = a.x_stride;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float4 wv = *reinterpret_cast<const float4*>(a.conv_w + (size_t)(ch + e) * 4);
            cwt[e][0] = wv.x; cwt[e][1] = wv.y; cwt[e][2] = wv.z; cwt[e][3] = wv.w;
            cbias[e] = a.conv_b ? a.conv_b[ch + e] : 0.0f;
        }
        if (tbeg == 0) {
            if (a.cstate_in) {
                const uint16_t* si = static_cast<const uint16_t*>(a.cstate_in) + (size_t)b * 3 * CD + ch;
                hw3 = *reinterpret_cast<const uint32_t*>(si);
                hw2 = *reinterpret_cast<const uint32_t*>(si + CD);
                hw1 = *reinterpret_cast<const uint32_t*>(si + 2 * CD);
            }
        } else {
            hw3 = *reinterpret_cast<const uint32_t*>(src + (size_t)(tbeg - 3) * cstride);
            hw2 = *reinterpret_cast<const uint32_t*>(src + (size_t)(tbeg - 2) * cstride);
            hw1 = *reinterpret_cast<const uint32_t*>(src + (size_t)(tbeg - 1) * cstride);
            if (docs) {
                const int d1 = docbase[tbeg - 1], d2 = docbase[tbeg - 2], d3 = docbase[tbeg - 3];
                pbits = (d1 != d2 ? 1 : 0) | (d2 != d3 ? 2 : 0);
            }
        }
        pbits = __builtin_amdgcn_readfirstlane(pbits);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            asm volatile("" : "+v"(cbias[e]));
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(cwt[e][j]));
        }
        asm volatile("" : "+v"(hw3), "+v"(hw2), "+v"(hw1));
    }

    const int nchunks = (tend - tbeg + Q - 1) / Q;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
        if (j < nchunks) {
            if (lead) issue_scalars(tbeg + j * Q, j);
            issue_tiles(tbeg + j * Q, j, 0, LD::NI_W);
        }
    }

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = tbeg + c * Q;
        const int st = NS == 2 ? (c & 1) : c % NS;
        const int cn = c + NS - 1;
        const int sn = NS == 2 ? (st ^ 1) : cn % NS;
        const unsigned char* sB = smem + st * LD::STAGE + LD::oB;
        const unsigned char* sX = smem + st * LD::STAGE + LD::oX + hh * LD::TX;
        float* sc = scal + (c & 1) * LD::SCW;
        // chunk c's copies have landed: only this wave's copies for chunks
        // c+1 .. c+NS-2 (dt / doc ids, then tiles, of each) may be newer
        if (c + NS - 2 < nchunks) wait_vmcnt_n((NS - 2) * (n_tiles + n_scal));
        else wait_vmcnt<0>();
        // ---- lead waves: segmented cumulative sum of dt*A (log2 domain) and the
        // chunk-state weights w_s = 2^(cs_end - cs_s) dt_s on the last segment
        if (lead) {
            const bool tok_ok = t0 + lane < tend;
            const unsigned char* dbuf = dbuf_of(st);
            float dtl = reinterpret_cast<const float*>(dbuf)[lane];
            const int d0 = reinterpret_cast<const int*>(dbuf)[Q + lane];
            const int d1 = reinterpret_cast<const int*>(dbuf)[2 * Q + lane];
            lds_wait();
            if (cn < nchunks) issue_scalars(t0 + (NS - 1) * Q, sn);
            if (CV) {
                const uint32_t wd = __float_as_uint(dtl);
                dtl = (h_l & 1) ? bf16_hi(wd) : bf16_lo(wd);
            }
            if (SP) dtl = softplus_f(dtl + dtbl);
            if (!tok_ok) dtl = 0.0f;
            const int bnd = (docs && tok_ok && t0 + lane > 0 && d0 != d1) ? 1 : 0;
            if (CV) {
                const uint64_t m = __ballot(bnd);
                if (lh == 0 && lane == 0) {
                    int* sci = reinterpret_cast<int*>(sc);
                    sci[LD::SC_ST] = (int)(uint32_t)m;
                    sci[LD::SC_ST + 1] = (int)(uint32_t)(m >> 32);
                    sci[LD::SC_ST + 2] = pbits;
                }
                pbits = (int)(m >> 63) | (int)((m >> 61) & 2);   // for the next chunk
            }
            float cs = dtl * A2l;
            int seg = bnd ? lane : -1;
            wave_segscan(cs, bnd, seg);
            const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
            const int last_seg = __builtin_amdgcn_readlane(seg, 63);
            const int wseg = last_seg >= 0 ? last_seg : 0;
            sc[lh * Q + lane] = lane >= wseg ? fast_exp2(cs_end - cs) * dtl : 0.0f;
            if (lane == 0) {
                sc[LD::SC_END + lh] = cs_end;
                if (lh == 0) reinterpret_cast<int*>(sc)[LD::SC_LAST] = last_seg;
            }
        }
        lds_barrier();                   // chunk c tiles + weights visible; chunk c-1 readers done
        // chunk cn's copies in two halves, the second after this wave's (w o X)
        // fragments: all waves issuing them at once would queue behind one
        // another in the CU's memory pipeline before their own compute
        constexpr int kHalfP = (LD::NI_W + 1) / 2;
        if (cn < nchunks) issue_tiles(t0 + (NS - 1) * Q, sn, 0, kHalfP);
        const float cs_end = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sc[LD::SC_END + hh])));
        const int last_seg = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(sc)[LD::SC_LAST]);
        const bool has_bnd = last_seg >= 0;

        if constexpr (CV) {
            // ---- conv + activation of the chunk's raw B and X tiles, in place
            // (the same pass as the main kernel's, without C)
            unsigned char* stg = smem + st * LD::STAGE;
            const int* sci = reinterpret_cast<const int*>(sc);
            const uint64_t smask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(sci[LD::SC_ST + 1]) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane(sci[LD::SC_ST]);
            const int r0 = cseg * CM::R;
            const bool more = c + 1 < nchunks;
            auto ldw = [&](int r) { return *reinterpret_cast<const uint32_t*>(stg + conv_off<RBU>(cw, r)); };
            uint32_t v3 = 0, v2 = 0, v1 = 0;
            int pb = 0;
            if (c_on) {
                if (cseg == 0) {
                    v3 = hw3; v2 = hw2; v1 = hw1;
                    pb = __builtin_amdgcn_readfirstlane(sci[LD::SC_ST + 2]);
                    if (more) { hw3 = ldw(Q - 3); hw2 = ldw(Q - 2); hw1 = ldw(Q - 1); }
                } else {
                    v3 = ldw(r0 - 3); v2 = ldw(r0 - 2); v1 = ldw(r0 - 1);
                    pb = (int)((smask >> (r0 - 1)) & 1) | (int)(((smask >> (r0 - 2)) & 1) << 1);
                }
            }
            lds_barrier();               // every raw halo row is read before any row is overwritten
            if (c_on) {
                if (pb & 1) { v3 = 0; v2 = 0; }
                if (pb & 2) v3 = 0;
                conv_rows<RBU>(stg, cw, r0, min(r0 + CM::R, Q), smask, v3, v2, v1, cwt, cbias, a.act == 0);
            }
            lds_barrier();               // the convolved tiles are visible
        }

        // ---- (w o X)^T fragments of this wave's blocks via transpose reads
        FragBF xw[PB][4];
        const float* wv = sc + hh * Q;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const float4 w = *reinterpret_cast<const float4*>(wv + 16 * sb + 4 * q4);
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const uint32_t xtr = SX::off(4 * q4 + j16 / 4, p0 + 16 * pb + 4 * (j16 % 4));
                const FragBF xf = tr_read(sX, xtr + 16 * sb * XB);
                xw[pb][sb].a = pack_bf16x2(w.x * bf16_lo(xf.a), w.y * bf16_hi(xf.a));
                xw[pb][sb].b = pack_bf16x2(w.z * bf16_lo(xf.b), w.w * bf16_hi(xf.b));
            }
        }
        if (cn < nchunks) issue_tiles(t0 + (NS - 1) * Q, sn, kHalfP, LD::NI_W);
        // ---- S = B^T (w o X) per block; H = dec H + S (dec = 0 past a document start)
        const float dec = has_bnd ? 0.0f : fast_exp2(cs_end);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint32_t btr = SB::off(4 * q4 + j16 / 4, 16 * nt + 4 * (j16 % 4));
            f32x4 acc[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; sb += 2) {
                const FragBF a0 = tr_read(sB, btr + 16 * sb * RB);
                const FragBF a1 = tr_read(sB, btr + 16 * (sb + 1) * RB);
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[pb] = mma_bf16(acc[pb], a0, a1, xw[pb][sb], xw[pb][sb + 1]);
            }
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) Hs[pb][nt][r] = fmaf(dec, Hs[pb][nt][r], acc[pb][r]);
        }
        log2dec += cs_end;
        reset = reset || has_bnd;
    }

    const size_t u = ((size_t)b * H + h) * (a.K - 1) + k;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
        float* hl = a.hloc + u * 64 * N + (size_t)(p0 + 16 * pb + j16) * N + 4 * q4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<float4*>(hl + 16 * nt) =
                make_float4(Hs[pb][nt][0], Hs[pb][nt][1], Hs[pb][nt][2], Hs[pb][nt][3]);
    }
    if (wave % WPH == 0 && lane == 0) a.dec[u] = reset ? -1.0f : fast_exp2(log2dec);   // the head's first wave
    if (k == 0 && a.h0) {
        // the main pass reads this copy instead of init_state
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            const size_t o = (((size_t)b * H + h) * 64 + p0 + 16 * pb + j16) * N + 4 * q4;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<float4*>(a.h0 + o + 16 * nt) =
                    *reinterpret_cast<const float4*>(a.init_state + o + 16 * nt);
        }
    }
}

// LDS layout of the full pass for N and HPW.  Two stages: copies one chunk
// ahead already cover the HBM latency (three- and four-stage rings measured
// no faster on the Mini-K3 and large-layer workloads) and leave the most LDS
// for resident workgroups.  z goes in the ring and M^T is split into halves
// where the layout fits a CU; otherwise z is single-buffered, then M^T is
// one bf16 rounding.  ok: some layout fits.
// One-time preparation of a kernel on the current device, before its first
// launch there: refuse a build whose kernel uses scratch (no_scratch: the
// kernel's explicit vector-memory waits count only its own copies, stores and
// loads, so register spills would add uncounted operations), and raise its
// dynamic-LDS cap to `lds`.  Thread-safe; each (kernel, device) pair is
// prepared once per process.
hipError_t prepare_kernel(const void* fn, size_t lds, bool no_scratch) {
    constexpr int kMaxDevices = 64;
    constexpr int kMaxKernels = 256;
    static std::mutex mu;
    static const void* fns[kMaxKernels] = {};
    static uint64_t ready[kMaxKernels] = {};   // bit d: prepared on device d
    static int nfns = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    int i = 0;
    while (i < nfns && fns[i] != fn) ++i;
    if (i < nfns && (ready[i] >> dev & 1)) return hipSuccess;
    if (no_scratch) {
        hipFuncAttributes fa;
        e = hipFuncGetAttributes(&fa, fn);
        if (e != hipSuccess) return e;
        if (fa.localSizeBytes != 0) return hipErrorInvalidDeviceFunction;
    }
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (i == nfns) {
        if (nfns == kMaxKernels) return hipSuccess;   // not remembered: prepared again next time
        fns[nfns++] = fn;
    }
    ready[i] |= uint64_t(1) << dev;
    return hipSuccess;
}

template <int N, int HPW>
struct BfPlan {
    static constexpr int NS = 2;
    static constexpr bool ZR = LdsBf<N, HPW, NS, true, true>::bytes <= 163840;
    static constexpr bool MS = ZR || LdsBf<N, HPW, NS, false, true>::bytes <= 163840;
    using LD = LdsBf<N, HPW, NS, ZR, MS>;
    static constexpr bool ok = LD::bytes <= 163840;
};
template <int N, bool SP, int HPW, bool CV>
hipError_t launch_scan_bf16_k(const ScanArgs& a, int units, hipStream_t stream) {
    using PL = BfPlan<N, HPW>;
    const void* fn = reinterpret_cast<const void*>(&ssd_scan_bf16_kernel<N, SP, HPW, CV, PL::NS, PL::ZR, PL::MS>);
    const size_t lds = PL::LD::bytes;
    if (hipError_t e = prepare_kernel(fn, lds, true); e != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_scan_bf16_kernel<N, SP, HPW, CV, PL::NS, PL::ZR, PL::MS>), dim3(units), dim3(256 * HPW),
                       lds, stream, a);
    return hipGetLastError();
}
template <int N, int HPW>
hipError_t launch_scan_bf16_full(const ScanArgs& a, int units, hipStream_t stream) {
    if (a.conv) return launch_scan_bf16_k<N, true, HPW, true>(a, units, stream);
    return a.dt_softplus ? launch_scan_bf16_k<N, true, HPW, false>(a, units, stream)
                         : launch_scan_bf16_k<N, false, HPW, false>(a, units, stream);
}
// the state-only pre-pass: PRE_HPW heads per workgroup, kPrePB channel blocks
// per wave (one with the fused conv, whose in-LDS pass wants every wave of a
// CU), kPreStages stages
constexpr int kPreStages = 3;
constexpr int kPrePB = 2;
template <int N, bool SP, int PRE_HPW, bool CV>
hipError_t launch_scan_state_k(const ScanArgs& a, hipStream_t stream) {
    constexpr int PB = CV ? 1 : kPrePB;
    using LD = LdsPre<N, PRE_HPW, PB, kPreStages>;
    const void* fn = reinterpret_cast<const void*>(&ssd_scan_state_kernel<N, SP, PRE_HPW, PB, kPreStages, CV>);
    if (hipError_t e = prepare_kernel(fn, LD::bytes, true); e != hipSuccess) return e;
    const int units = a.B * (a.H / PRE_HPW) * (a.K - 1);
    hipLaunchKernelGGL((ssd_scan_state_kernel<N, SP, PRE_HPW, PB, kPreStages, CV>), dim3(units), dim3(64 * LD::NW),
                       LD::bytes, stream, a);
    return hipGetLastError();
}
template <int N, int PRE_HPW>
hipError_t launch_scan_bf16_pre(const ScanArgs& a, hipStream_t stream) {
    if (a.conv) return launch_scan_state_k<N, true, PRE_HPW, true>(a, stream);
    return a.dt_softplus ? launch_scan_state_k<N, true, PRE_HPW, false>(a, stream)
                         : launch_scan_state_k<N, false, PRE_HPW, false>(a, stream);
}
template <int N, int HPW>
hipError_t launch_scan_bf16(const ScanArgs& a, int pre_hpw, hipStream_t stream) {
    if (a.K > 1) {
        hipError_t e = pre_hpw == 4 ? launch_scan_bf16_pre<N, 4>(a, stream)
                     : pre_hpw == 2 ? launch_scan_bf16_pre<N, 2>(a, stream)
                                    : launch_scan_bf16_pre<N, 1>(a, stream);
        if (e != hipSuccess) return e;
    }
    return launch_scan_bf16_full<N, HPW>(a, a.B * (a.H / HPW) * a.K, stream);
}

template <typename T, int N, int MODE, int HPW>
hipError_t launch_scan_mode(const ScanArgs& a, hipStream_t stream) {
    const size_t lds = Lds<N, MODE, HPW>::bytes;
    if (hipError_t e = prepare_kernel(reinterpret_cast<const void*>(&ssd_scan_kernel<T, N, MODE, HPW>), lds, false);
        e != hipSuccess)
        return e;
    const int units = a.B * (a.H / HPW) * (MODE == kFull ? a.K : a.K - 1);
    hipLaunchKernelGGL((ssd_scan_kernel<T, N, MODE, HPW>), dim3(units), dim3(256 * HPW), lds, stream, a);
    return hipGetLastError();
}
template <typename T, int N, int HPW>
hipError_t launch_scan_f32(const ScanArgs& a, hipStream_t stream) {
    if (a.K > 1) {
        hipError_t e = launch_scan_mode<T, N, kStateOnly, HPW>(a, stream);
        if (e != hipSuccess) return e;
    }
    return launch_scan_mode<T, N, kFull, HPW>(a, stream);
}

// ---- bf16 plan: heads per workgroup, then the sequence split.
constexpr int kCUs = 256;
constexpr size_t kLdsPerCU = 163840;
constexpr int kMaxWavesPerCU = 32;

template <int N>
size_t bf16_lds_n(int hpw, bool full) {
    if (full) {
        switch (hpw) {
            case 1: return BfPlan<N, 1>::LD::bytes;
            case 2: return BfPlan<N, 2>::LD::bytes;
            case 4: return BfPlan<N, 4>::LD::bytes;
        }
    } else {
        switch (hpw) {
            case 1: return LdsPre<N, 1, kPrePB, kPreStages>::bytes;
            case 2: return LdsPre<N, 2, kPrePB, kPreStages>::bytes;
            case 4: return LdsPre<N, 4, kPrePB, kPreStages>::bytes;
        }
    }
    return kLdsPerCU + 1;
}
size_t bf16_lds(int N, int hpw, bool full) {
    switch (N) {
        case 16: return bf16_lds_n<16>(hpw, full);
        case 32: return bf16_lds_n<32>(hpw, full);
        case 64: return bf16_lds_n<64>(hpw, full);
        case 128: return bf16_lds_n<128>(hpw, full);
    }
    return kLdsPerCU + 1;
}
// workgroups of 4 hpw waves that fit one CU by LDS
int bf16_wgs_per_cu(int N, int hpw, bool full) {
    const size_t bytes = bf16_lds(N, hpw, full);
    if (bytes > kLdsPerCU) return 0;
    const int waves = full ? 4 * hpw : 4 * hpw / kPrePB;
    return (int)std::min<size_t>(kLdsPerCU / bytes, (size_t)(kMaxWavesPerCU / waves));
}
// Heads per workgroup: the largest of 4, 2, 1 that divides the heads of a
// group and gives the most waves per CU.
int bf16_hpw(int N, int H, int G) {
    const int hg = H / G;
    int best = 1, best_waves = 0;
    for (int hpw : {4, 2, 1}) {
        if (hg % hpw) continue;
        const int waves = bf16_wgs_per_cu(N, hpw, true) * 4 * hpw;
        if (waves > best_waves) { best_waves = waves; best = hpw; }
    }
    return best;
}
// Heads per workgroup of the state-only pre-pass: the largest that divides the
// heads of a group and keeps at least PRE_MIN_WAVES waves per CU.
int bf16_pre_hpw(int N, int H, int G) {
    const int hg = H / G;
    for (int hpw : {4, 2, 1})
        if (hg % hpw == 0 && bf16_wgs_per_cu(N, hpw, false) > 0) return hpw;
    return 1;
}

// fp32 heads per workgroup: two where the heads of a group pair up (the plan
// fits a CU at every supported N), else one.
int f32_hpw(int H, int G) { return (H / G) % 2 == 0 ? 2 : 1; }

template <typename T, int N>
hipError_t launch_scan_n(const ScanArgs& a, hipStream_t stream) {
    if constexpr (!std::is_same<T, float>::value) {
        const int pre = bf16_pre_hpw(N, a.H, a.G);
        switch (bf16_hpw(N, a.H, a.G)) {
            case 4:
                if constexpr (BfPlan<N, 4>::ok) return launch_scan_bf16<N, 4>(a, pre, stream);
                return hipErrorInvalidConfiguration;   // not chosen: bf16_hpw sees no room for 4 heads
            case 2: return launch_scan_bf16<N, 2>(a, pre, stream);
            default: return launch_scan_bf16<N, 1>(a, pre, stream);
        }
    } else {
        return f32_hpw(a.H, a.G) == 2 ? launch_scan_f32<T, N, 2>(a, stream) : launch_scan_f32<T, N, 1>(a, stream);
    }
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

// Sequence split.  fp32: enough (b, h, superchunk) units to give every CU
// several workgroups, with superchunks of at least 8 chunks.  bf16: the K
// (at most 8) that minimises the critical path in chunk steps -- rounds of
// resident workgroups times chunks per superchunk -- counting the state-only
// pre-pass at 0.4 of a full chunk step.
void scan_split(int B, int L, int H, int N, int G, int dtype, int& K, int& S) {
    const int nch = (L + Q - 1) / Q;
    if (nch <= 1) { K = 1; S = Q * std::max(nch, 1); return; }
    int k = 1;
    if (dtype == 0) {   // fp32
        constexpr long kTargetUnits = 1024;   // 4 workgroups per CU on 256 CUs
        constexpr int kMinChunks = 8;
        const long wgs = (long)B * (H / f32_hpw(H, G));
        while (wgs * k < kTargetUnits && nch / (2 * k) >= kMinChunks) k *= 2;
    } else {
        const int hpw = bf16_hpw(N, H, G);
        const long units = (long)B * (H / hpw);
        const long slots = (long)kCUs * std::max(bf16_wgs_per_cu(N, hpw, true), 1);
        const int pre_hpw = bf16_pre_hpw(N, H, G);
        const long units_pre = (long)B * (H / pre_hpw);
        const long slots_pre = (long)kCUs * std::max(bf16_wgs_per_cu(N, pre_hpw, false), 1);
        double best = 1e300;
        for (int kk = 1; kk <= 8 && kk <= nch; ++kk) {
            const int per = (nch + kk - 1) / kk;
            const int kr = (nch + per - 1) / per;      // superchunks actually used
            if (kr != kk) continue;
            double cost = (double)((units * kk + slots - 1) / slots) * per;
            if (kk > 1) cost += 0.4 * (double)((units_pre * (kk - 1) + slots_pre - 1) / slots_pre) * per;
            if (cost < best - 1e-9) { best = cost; k = kk; }
        }
    }
    const int per = (nch + k - 1) / k;           // chunks per superchunk
    K = (nch + per - 1) / per;
    S = per * Q;
}

// Static scratch of the no-allocation scan entry point: the split workspace
// (local end states, decays, the copy of init_state) of one call at a time
// per GPU.  In host code the array's name is only a stand-in for the symbol;
// its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = SSD_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t scan_static_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kStaticScratchBytes;
    return hipSuccess;
}

size_t scan_workspace_bytes(int B, int L, int H, int P, int N, int G, int dtype) {
    int K, S;
    scan_split(B, L, H, N, G, dtype, K, S);
    if (K <= 1) return 0;
    const size_t u = (size_t)B * H * (K - 1);
    // hloc [u][P][N], dec [u] (padded to 256 bytes), the copy of init_state [B][H][P][N]
    return u * (size_t)P * N * sizeof(float) + ((u * sizeof(float) + 255) / 256) * 256 +
           (size_t)B * H * P * N * sizeof(float);
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 0 ? launch_scan_t<float>(a, stream) : launch_scan_t<uint16_t>(a, stream);
}

}  // namespace ssd
