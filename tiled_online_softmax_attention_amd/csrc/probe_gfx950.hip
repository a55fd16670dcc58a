// probe_gfx950.hip -- sustained-rate probe of the bf16 matrix-core
// instruction the attention kernels are built from
// (v_mfma_f32_32x32x16_bf16).  It is a measurement aid, not part of the
// attention path: it gives the rate the chip holds for this instruction over
// long launches, which depends on the operand data (random operands draw more
// power than repeated constant ones, and the engine clock drops to stay
// within the power limit).  The attention kernels' roofline fraction is
// quoted against the published peak; this probe says how much of that peak
// is reachable at all on real data.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "probe_internal.h"

namespace attn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Each lane loads 8 A and 8 B fragments (fragment t*16 + i, wrapped by the
// power-of-two mask) and runs `iters` MFMAs per wave in four independent
// accumulation chains, taking a different (A, B) pair every instruction so
// that the operand bits change as they do in a real contraction.
//
// PAD 4-byte s_nop instructions in front of the loop move it through 16
// placements in instruction memory.  A loop made of nothing but MFMAs issues
// at a rate that depends on that placement (measured on MI355X: 1.36 to 1.82
// PFLOP/s for this loop on random operands, the same instructions shifted by
// multiples of 4 bytes), so the caller tries every placement and keeps the
// best; loops that mix MFMAs with other instructions, like the attention
// kernels', showed no such dependence (aligning their loops to 64, 128 or
// 256 bytes left the causal prefill within 0.4 %).
template <int PAD>
__global__ __launch_bounds__(256) void mfma_probe_kernel(const bf16x8_t* __restrict__ frag, uint32_t mask,
                                                         float* __restrict__ out, int iters)
{
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = frag[(t * 16u + (uint32_t)i) & mask];
        b[i] = frag[(t * 16u + 8u + (uint32_t)i) & mask];
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
#pragma unroll
    for (int p = 0; p < PAD; ++p) asm volatile("s_nop 0");
    for (int it = 0; it < iters / 32; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + 1) & 7], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 3) & 7], b[(k + 5) & 7], c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 5) & 7], b[(k + 2) & 7], c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 6) & 7], b[(k + 7) & 7], c3, 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[t] = s;
}

}  // namespace

int launch_mfma_probe(const void* fragments, int n_fragments, float* out, int blocks, int iters, int placement,
                      hipStream_t stream)
{
    typedef void (*probe_fn)(const bf16x8_t*, uint32_t, float*, int);
    static const probe_fn kernels[kProbePlacements] = {
        mfma_probe_kernel<0>,  mfma_probe_kernel<1>,  mfma_probe_kernel<2>,  mfma_probe_kernel<3>,
        mfma_probe_kernel<4>,  mfma_probe_kernel<5>,  mfma_probe_kernel<6>,  mfma_probe_kernel<7>,
        mfma_probe_kernel<8>,  mfma_probe_kernel<9>,  mfma_probe_kernel<10>, mfma_probe_kernel<11>,
        mfma_probe_kernel<12>, mfma_probe_kernel<13>, mfma_probe_kernel<14>, mfma_probe_kernel<15>};
    hipLaunchKernelGGL(kernels[placement], dim3((unsigned)blocks), dim3(256), 0, stream, (const bf16x8_t*)fragments,
                       (uint32_t)(n_fragments - 1), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace attn
