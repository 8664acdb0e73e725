// ssd_launch.hpp -- host-side argument blocks and launchers of the kernels.
// Arguments are already validated by api.cpp; sizes are in elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

struct ConvArgs {
    int B, L, C, H, dtype, act;
    // rows between batch rows: of raw, dt_raw and doc (Lb_in), of out and
    // dt_out (Lb_out); both >= L, and L for the public calls
    int Lb_in, Lb_out;
    const void* raw; int64_t raw_stride;
    const float* w; const float* bias;
    const void* dt_raw; int64_t dt_stride;
    const float* dt_bias;
    const int32_t* doc;
    const void* state_in; void* state_out;
    void* out; int64_t out_stride;
    float* dt_out;
};

struct ScanArgs {
    int B, L, H, P, N, G, dtype;
    int Lb;   // rows between batch rows of every [B][L][...] tensor (>= L; L for the public calls)
    const void* x; int64_t x_stride;
    const void* Bm; int64_t B_stride;
    const void* Cm; int64_t C_stride;
    const float* dt; int64_t dt_stride;
    int dt_softplus; const float* dt_bias;
    const float* A; const float* D;
    const void* z; int64_t z_stride;
    const int32_t* doc;
    const float* init_state; float* final_state;
    float* y; int64_t y_stride;
    // sequence split: K superchunks of S tokens (S a multiple of 64); K = 1 is
    // one sequential pass.  hloc / dec: workspace for the K-1 local states.
    int K, S;
    float* hloc; float* dec;
    // K > 1 with an initial state: the pre-pass copies init_state here and the
    // main pass reads the copy, so final_state may alias init_state even though
    // superchunk K-1 can finish before superchunk 0 starts.
    float* h0;
    // Fused conv prologue (bf16 only; the mixer entry point): x, Bm and Cm are
    // the raw column slices of one [x | B | C] tensor (conv_dim wide) and are
    // convolved (k = 4, weights [conv_dim][4]) and activated on chip; dt16 is
    // the raw bf16 dt, taken through softplus(dt16 + dt_bias).  conv = 0: off.
    int conv, act;
    const float* conv_w; const float* conv_b;
    const void* cstate_in; void* cstate_out;   // [B][3][conv_dim]
    const uint16_t* dt16; int64_t dt16_stride;
    // fp32 kernel: rows before y_row0 need no output (chunk-resume decode
    // reruns the working chunk for its newest rows only); their y is left as
    // it was.  0 for every public scan call.
    int y_row0;
};

struct StepArgs {
    int B, H, P, N, G, dtype, act;
    const void* xbc_raw; const void* dt_raw; const void* z;
    const float* conv_w; const float* conv_b; const float* dt_bias;
    const float* A; const float* D;
    void* conv_state; float* ssm_state; float* y;
};

// Mamba-1 selective scan: per (b, d) a diagonal state of N entries with
// decay exp(dt A[d][n]); B and C are shared by all channels of a token.
struct S6Args {
    int B, L, D, N, dtype;
    const void* x; int64_t x_stride;     // [B][L][D] (dtype)
    const void* dt; int64_t dt_stride;   // [B][L][D] (dtype)
    int dt_softplus; const float* dt_bias;
    const float* A;                      // [D][N]
    const void* Bm; int64_t B_stride;    // [B][L][N] (dtype), rows 16-byte aligned
    const void* Cm; int64_t C_stride;
    const float* D_skip;                 // [D] or null
    const void* z; int64_t z_stride;     // [B][L][D] (dtype) or null
    const int32_t* doc;                  // [B][L] or null
    const float* init_state; float* final_state;   // [B][D][N]
    float* y; int64_t y_stride;          // [B][L][D] fp32
    // sequence split (K superchunks of S tokens); workspace for K > 1:
    // hloc [B][D][K-1][N], sdt [B][D][K-1], h0 [B][D][N] (init_state copy)
    int K, S;
    float* hloc; float* sdt; float* h0;
};

// Backward (VJP) of the chunked scan for a zero initial state.  Inputs as in
// ScanArgs (dt fp32: activated, or raw with dt_softplus); gy = dLoss/dy.
// Outputs fp32; dB / dC are summed over a group's heads.
struct BwdArgs {
    int B, L, H, P, N, G, dtype;
    const void* x; int64_t x_stride;
    const void* Bm; int64_t B_stride;
    const void* Cm; int64_t C_stride;
    const float* dt; int64_t dt_stride;
    // dt_softplus = 1: dt is raw and dt := softplus(dt + dt_bias); ddt is then
    // with respect to the raw value.  chain_from_dt = 1 (dt_softplus = 0): dt
    // is softplus(v) of some v and ddt is with respect to v, using
    // softplus'(v) = 1 - exp(-dt).
    int dt_softplus, chain_from_dt; const float* dt_bias;
    const float* A; const float* D;
    const void* z; int64_t z_stride;
    const int32_t* doc;
    const float* gy; int64_t gy_stride;
    float* dx; int64_t dx_stride;
    float* dB; int64_t dB_stride;
    float* dC; int64_t dC_stride;
    float* ddt; int64_t ddt_stride;
    float* dz; int64_t dz_stride;
    float* ddt_bias; float* dA; float* dD;   // [H] or null
    // workspace: nc chunks of 64 tokens
    int nc;
    float* S;      // [B][H][nc][N][P]  chunk-local states, then the state entering each chunk
    float* dS;     // [B][H][nc][N][P]  chunk adjoint inputs, then the adjoint of the state leaving each chunk
    float* dec;    // [B][H][nc]        decay across each chunk (0 where a document starts in it)
    float* part;   // [3][B * nc][H]    per-chunk partial sums of dA, dD and ddt_bias
};

// Backward of the conv (zero conv state): dout = dLoss/d(conv output) fp32.
struct ConvBwdArgs {
    int B, L, C, dtype, act;
    const void* raw; int64_t raw_stride;
    const float* w; const float* bias;
    const int32_t* doc;
    const float* dout; int64_t dout_stride;
    float* draw; int64_t draw_stride;
    float* dw; float* dbias;               // [C][4], [C] (dbias may be null)
    int ntc;                               // token chunks of 64
    float* part;                           // [B * ntc][C][5] per-chunk partial sums of dw and dbias
};

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);
// Sequence split chosen for these sizes (1 = none) and its superchunk length.
void scan_split(int B, int L, int H, int N, int G, int dtype, int& K, int& S);
size_t scan_workspace_bytes(int B, int L, int H, int P, int N, int G, int dtype);
// The scan's file-scope static scratch on the current device: its address,
// looked up once per device (hipGetSymbolAddress) and cached; *bytes = its
// size.  Allocates nothing.
hipError_t scan_static_scratch(void** ptr, size_t* bytes);
hipError_t launch_step(const StepArgs& a, hipStream_t stream);
// Copies n 16-byte words src -> dst (src == nullptr: zero fill); used for the
// L = 0 state pass-through without a memset node.
hipError_t launch_copy16(const void* src, void* dst, size_t n, hipStream_t stream);
// Copies rows of row_bytes (a multiple of 16) for B batch rows x `rows` rows:
// src/dst row r of batch b at base + b * batch_stride + r * row_stride (bytes).
hipError_t launch_copy_rows(const void* src, int64_t src_row_stride, int64_t src_batch_stride, void* dst,
                            int64_t dst_row_stride, int64_t dst_batch_stride, int B, int rows, int row_bytes,
                            hipStream_t stream);

size_t step_lds_bytes(int H, int P, int N, int G);
// Ragged batches: rows t >= lengths[b] of y (fp32, width a multiple of 4,
// rows 16-byte aligned) set to +0.0.
hipError_t launch_zero_rows(float* y, int64_t stride, int B, int L, int width, const int32_t* lengths,
                            hipStream_t stream);

hipError_t launch_s6(const S6Args& a, hipStream_t stream);

size_t scan_bwd_workspace_bytes(int B, int L, int H, int P, int N);
hipError_t launch_scan_bwd(const BwdArgs& a, hipStream_t stream);
size_t conv_bwd_workspace_bytes(int B, int L, int C);
// Zero fill of n floats by a kernel (no memset node).
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream);
hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t stream);
void s6_split(int B, int L, int D, int& K, int& S);
size_t s6_workspace_bytes(int B, int L, int D, int N);

}  // namespace ssd
