// gdn_launch.h -- internal launchers shared by the C ABI (api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Workspace carve-up of the chunked prefill; every region is 256-byte aligned.
// E is the operand type (float16 for bf16 inputs, float32 for float32 inputs).
struct PrefillWorkspace {
    float *tok;     // [B*Hv*NC][2][64]: gamma = e^G by token, then token 16r+m at 4m+r
    void *apair;    // [B*Hv*NC][6][64 lanes][8] E: diag(eta) (I+L)^{-1} diag(beta) operand fragments
    void *qpair;    // [B*Hv*NC][6][64 lanes][8] E: A_qk (I+L)^{-1} diag(beta) operand fragments
    void *qimg;     // [B*Hk*NC][64][Dk] E: Q tile images
    void *kimg;     // [B*Hk*NC][64][Dk] E: K tile images
    void *timg;     // [B*Hk*NC][Dk][64] E: K^T tile images (float32 operands only)
    size_t bytes;   // total
};

size_t prefill_workspace_layout(int B, int T, int Hk, int Hv, int Dk, bool f32, void *base,
                                PrefillWorkspace *ws);

struct PrefillArgs {
    int B, T, Hk, Hv, Dk, Dv;
    bool f32;
    float scale;
    const void *q, *k, *v;
    const float *a, *b, *A_log, *dt_bias;
    const float *S0;
    void *out;
    float *ST;
};

hipError_t launch_chunk_local(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s);
hipError_t launch_state_scan(const PrefillArgs &p, const PrefillWorkspace &ws, hipStream_t s);
hipError_t launch_state_copy(const PrefillArgs &p, hipStream_t s);  // T == 0: S_T = S_0 (or 0)

// Workspace of the Gated DeltaNet-2 chunked prefill (bfloat16 inputs, float16
// operands), per (sequence, value head, chunk) unit; every region 256-byte
// aligned.  G is the in-chunk inclusive prefix of the channel-wise log decay.
// Element type E: float16 for bfloat16 inputs, float32 for float32 inputs.
struct Gdn2Workspace {
    void *eimg;    // [B*Hv*NC][64][Dk] E image: (sigmoid(erase) . k) . e^{G}
    void *khimg;   // [B*Hv*NC][64][Dk] E image: k . e^{G_C - G}
    void *qimg;    // [B*Hv*NC][64][Dk] E image: scale q . e^{G}
    void *khtimg;  // [B*Hv*NC][Dk][64] f32 image of Kh^T (float32 only; the float16
                   // scan reads Kh^T operands from the Kh image with transposed LDS reads)
    void *apair;   // [B*Hv*NC][6][64 lanes][8] E: A = (I + M)^{-1} operand fragments
    void *qpair;   // [B*Hv*NC][6][64 lanes][8] E: A_qk A operand fragments
    float *gc;     // [B*Hv*NC][Dk] f32: e^{G_C} per key channel
    void *z;       // [B,T,Hv,Dv] E: sigmoid(write) . v
    size_t bytes;  // total
};

size_t gdn2_workspace_layout(int B, int T, int Hv, int Dk, int Dv, bool f32, void *base, Gdn2Workspace *ws);

struct Gdn2Args {
    int B, T, Hk, Hv, Dk, Dv;
    bool f32;
    float scale;
    const void *q, *k, *v, *a, *erase, *write;  // bfloat16 or float32
    const float *A_log;                          // [Hv][Dk]
    const float *S0;
    void *out;
    float *ST;
};

hipError_t launch_chunk_local2(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s);
hipError_t launch_chunk_local2_f32(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s);
hipError_t launch_state_scan2(const Gdn2Args &p, const Gdn2Workspace &ws, hipStream_t s);

// Gradient of the Gated DeltaNet-2 chunked forward (bwd2.hip).  Float32
// workspace, per (sequence, value head, chunk) unit u unless noted.
struct Bwd2Workspace {
    float *A, *Aq;                 // [U][64][64]: (I + M)^{-1}; A_qk (scale folded into q)
    float *Et, *Qt, *Kh;           // [U][64][Dk]: e^{G} e, e^{G} scale q, e^{G_C - G} k
    float *gC;                     // [U][Dk]: e^{G_C}
    float *U, *R, *dU, *dR;        // [U][64][Dv]
    float *Sn, *dS1;               // [U][Dk][Dv]: state before the chunk; its gradient after
    float *dEt, *dQt, *dKh;        // [U][64][Dk]
    float *dgC;                    // [U][Dk]
    float *dM, *dAq;               // [U][64][64]
    float *dqh, *dkh;              // [B][T][Hv][Dk]: per value head, summed per key head later
    float *dAl;                    // [U][Dk]: per-chunk part of dA_log
    size_t bytes;
};

size_t bwd2_workspace_layout(int B, int T, int Hv, int Dk, int Dv, void *base, Bwd2Workspace *ws);

struct Bwd2Args {
    int B, T, Hk, Hv, Dk, Dv, NC;
    bool f32;                                    // float32 inputs (else bfloat16)
    float scale;
    const void *q, *k, *v, *a, *erase, *write;  // input type
    const float *A_log, *S0;
    const void *dout;                            // input type, [B,T,Hv,Dv]
    const float *dST;                            // [B,Hv,Dk,Dv] or null
    float *dq, *dk, *dv, *da, *derase, *dwrite, *dA_log, *dS0;
};

// ev: null, or 7 events recorded before each of the six launches and after the last
hipError_t launch_bwd2(const Bwd2Args &p, const Bwd2Workspace &ws, hipStream_t s, const hipEvent_t *ev);

// One recurrent step.  The scalar decay (gdn2 = false): a, b [B,H_v] float32,
// A_log, dt_bias [H_v].  The channel-wise decay (gdn2 = true): a, b = erase
// [B,H_v,d_k] and write [B,H_v,d_v] in the input type, A_log [H_v,d_k].
struct DecodeArgs {
    int B, Hk, Hv, Dk, Dv;
    bool f32, gdn2;
    float scale;
    const void *q, *k, *v;
    const void *a, *b, *write;
    const float *A_log, *dt_bias;
    float *state;
    void *out;
};

hipError_t launch_decode(const DecodeArgs &p, hipStream_t s);

// Gated RMS normalisation of rows x d values (d = 64 or 128).
struct NormArgs {
    long long rows;
    int d;
    bool f32, silu;
    float eps;
    const void *x, *z;
    const float *w;
    void *out;
};
hipError_t launch_gated_rmsnorm(const NormArgs &p, hipStream_t s);

// Depthwise causal conv1d (+ SiLU) over x [B,T,C] (C = 2 qk + v channels),
// split into q, k [B,T,qk] and v [B,T,C - 2 qk]; state / state_out [B][K-1][C]
// or null (state_out may be state).
struct ConvArgs {
    int B, T, C, qk, K;
    bool f32, silu;
    const void *x;
    const float *w, *bias;
    const void *state;
    void *state_out, *q, *k, *v;
};
hipError_t launch_causal_conv1d(const ConvArgs &p, hipStream_t s);
int conv_tokens_per_block();
long long gated_rmsnorm_max_rows();

}  // namespace gdn
