// Internal interface between the host entry points (wkv7_api.hip) and the
// kernel launchers of librwkv7_wkv.so.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rwkv7_wkv.h"

namespace wkv7 {

constexpr int kN = 64;  // head size of the chunked kernels (the scan and decode also take 128)
extern const bool kChunkedAvailable;

struct EpilogueArgs {
    const float *ln_w;  // [H*N] or nullptr (= 1)
    const float *ln_b;  // [H*N] or nullptr (= 0)
    const float *r_k;   // [H*N]
    float eps;
};

struct ForwardArgs {
    const void *r, *w, *k, *v, *kappa, *a;  // [B,T,H,N] in dt
    const float *s0;                        // [B,H,N,N] or nullptr (zero state)
    void *y;                                // [B,T,H,N] in dt
    float *s_out;                           // [B,H,N,N] or nullptr
    int B, T, H;
    int N;  // head size: 64 or 128
    bool bf16;
    bool w32;  // bf16 inputs except w, which is float32
    bool epilogue;
    EpilogueArgs epi;
    void *workspace;
    size_t workspace_bytes;
    float *s_ckpt;  // [B,H,ceil(T/kCkpt),N,N]: state before every kCkpt-th token, or nullptr
    // bidirectional calls: the reverse pass walks tokens T-1 .. 0 and writes its
    // readouts as float32 to y_f32 (no epilogue); the forward pass adds y_add to
    // its readouts before the epilogue.  Both [B,T,H,N] float32, or nullptr.
    bool reverse;
    float *y_f32;
    const float *y_add;
    // fused time-mix prologue: k holds the raw keys, kappa is unused; the kernels
    // form kappa = normalise(k * k_k) and k <- k + k (a-1) k_a, and multiply the
    // readouts (after the epilogue) by the gate g when it is given
    bool fused;
    const float *k_k, *k_a;  // [H*N]
    const void *g;           // [B,T,H,N] in dt, or nullptr
};

constexpr int kCkpt = RWKV7_CKPT_INTERVAL;  // tokens between stored states

struct BackwardArgs {
    const void *r, *w, *k, *v, *kappa, *a;  // [B,T,H,N] in dt (forward inputs)
    const void *dy;                         // [B,T,H,N] in dt
    const float *s_ckpt;                    // [B,H,ceil(T/kCkpt),N,N]
    const float *ds_T;                      // [B,H,N,N] or nullptr (zero)
    void *dr, *dw, *dk, *dv, *dkappa, *da;  // [B,T,H,N] in dt
    float *ds0;                             // [B,H,N,N] or nullptr
    int B, T, H;
    int N;  // head size: 64, or 128 (token-by-token kernel only)
    bool bf16;
    uint16_t *ds_ws;  // chunked: per (b, h, chunk) the bf16 dS_C diag(g_C), 8 KiB in lane order
    float *scan_ws;   // token-by-token at N = 128: partial column sums and the carried cotangent
    bool w32;      // w and dw float32 (the other vectors bf16)
};

struct DecodeArgs {
    const void *r, *w, *k, *v, *kappa, *a;  // [B,H,N] in dt
    float *state;                           // [B,H,N,N], in place
    void *y;                                // [B,H,N] in dt
    int B, H;
    int N;                                  // head size: 64 or 128
    bool bf16;
    bool w32;  // bf16 inputs except w, which is float32
    bool epilogue;
    EpilogueArgs epi;
    // fused time-mix prologue (as in ForwardArgs): k raw, kappa unused
    bool fused;
    const float *k_k, *k_a;  // [H*N]
    const void *g;           // [B,H,N] in dt, or nullptr
};

// Each launcher enqueues its kernels on `stream` and returns hipSuccess or the
// launch error.  Arguments were validated by the caller.
hipError_t launch_scan(const ForwardArgs &p, hipStream_t stream);
hipError_t launch_chunked(const ForwardArgs &p, hipStream_t stream);
size_t chunked_workspace_bytes(int B, int T, int H);
hipError_t launch_decode(const DecodeArgs &p, hipStream_t stream);
// token-by-token backward (f32, bf16, bf16 with float32 w; head size 64 or 128);
// at 128 it needs scan_ws of the size below (0 at 64)
hipError_t launch_backward(const BackwardArgs &p, hipStream_t stream);
size_t backward_scan_workspace_bytes(int B, int T, int H, int N);
// chunked backward (bf16, head size 64): reverse chain over the chunks, then
// every chunk's gradients in parallel; needs ds_ws of the size below
hipError_t launch_backward_chunked(const BackwardArgs &p, hipStream_t stream);
size_t backward_chunked_workspace_bytes(int B, int T, int H);
// whether the chunked backward's launch grids fit (B*H workgroups, and B*H
// times the number of 8-chunk groups)
bool backward_chunked_grid_ok(int B, int T, int H);
// S_T for T == 0: copy s0 (or zeros) into s_out.
hipError_t launch_state_copy(const float *s0, float *s_out, size_t count, hipStream_t stream);

}  // namespace wkv7
