// bwd_internal.h -- argument block and launcher of the attention backward,
// shared between the C-ABI host code (attn_api.hip) and bwd_gfx950.hip.
// Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct BwdArgs {
    const void* q;       // [B, H, N, d] bf16
    const void* k;       // [B, H_kv, N, d] bf16
    const void* v;       // [B, H_kv, N, d] bf16
    const void* o;       // [B, H, N, d] bf16, the forward output
    const float* lse;    // [B, H, N], the forward log-sum-exp (natural log)
    const void* dout;    // [B, H, N, d] bf16, gradient of the output
    void* dq;            // [B, H, N, d] bf16
    void* dk;            // [B, H_kv, N, d] bf16
    void* dv;            // [B, H_kv, N, d] bf16
    float* ws;           // [B * H][2][N] fp32: lse * log2 e of each query row, then D = dO . O
    int B, H, H_kv, N, d;
    float scale;
    int causal;
    int pair_q;          // dQ workgroups take query tiles t and n-1-t: -1 when causal, 0 no, 1 yes
    int pair_kv;         // dK/dV workgroups take key blocks kb and nkb-1-kb: -1 when causal, 0 no, 1 yes
};

inline size_t bwd_workspace_bytes(int B, int H, int N)
{
    return (size_t)B * (size_t)H * (size_t)N * 2u * sizeof(float);
}

// 0 on success, -1 launch failure, -2 grid too large.
int launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace attn
