// coexec_probe.hip -- measurement support, not part of the attention library:
// whether matrix work of one wave and vector work of another wave on the same
// SIMD overlap in time.  One workgroup of 512 threads per CU (eight waves, two
// per SIMD): waves 0-3 issue eight independent chains of
// v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs or in arch VGPRs), waves 4-7
// issue sixteen independent chains of FMA followed by exp2 (or by a second
// FMA).  `mode` bit 0 lets the matrix waves work, bit 1 the vector waves;
// timing modes 1, 2 and 3 gives the overlap.  Results are only folded into
// `out` (one float per thread) so that nothing is optimised away; the values
// carry no meaning.  Built into libswa_measure.so (C ABI below).
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int AGPR, int TRANS>
__global__ __launch_bounds__(512) void coexec_kernel(float *out, int iters_m, int iters_v,
                                                     int mode) {
    const int tid = threadIdx.x, wave = tid >> 6;
    float r = 0.f;
    if (wave < 4) {
        if (mode & 1) {
            bf16x8 a, b;
            for (int i = 0; i < 8; i++) {
                a[i] = (__bf16)(0.001f * (tid + i));
                b[i] = (__bf16)(0.002f * i);
            }
            f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
            for (int it = 0; it < iters_m; it++) {
                // the accumulator's register file is chosen by the constraint
                // ("a": AGPRs, "v": arch VGPRs); the builtin lets the compiler pick
                if (AGPR) {
#define SWA_M(c) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b))
                    SWA_M(c0); SWA_M(c1); SWA_M(c2); SWA_M(c3);
                    SWA_M(c4); SWA_M(c5); SWA_M(c6); SWA_M(c7);
#undef SWA_M
                } else {
#define SWA_M(c) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b))
                    SWA_M(c0); SWA_M(c1); SWA_M(c2); SWA_M(c3);
                    SWA_M(c4); SWA_M(c5); SWA_M(c6); SWA_M(c7);
#undef SWA_M
                }
            }
            // the accumulators are read only after the last chain has drained
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            for (int e = 0; e < 16; e++)
                r += c0[e] + c1[e] + c2[e] + c3[e] + c4[e] + c5[e] + c6[e] + c7[e];
        }
    } else if (mode & 2) {
        float x[16];
        for (int j = 0; j < 16; j++) x[j] = 0.01f * (tid + j);
        const float c = 0.999f, d = -0.5f;
        for (int it = 0; it < iters_v; it++) {
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const float y = fmaf(x[j], c, d);
                x[j] = TRANS ? __builtin_amdgcn_exp2f(y) : fmaf(y, c, d);
            }
        }
        for (int j = 0; j < 16; j++) r += x[j];
    }
    out[blockIdx.x * 512 + tid] = r;
}

}  // namespace

// out: device float[blocks * 512]; iters_m / iters_v: chain lengths of the
// matrix and vector waves; mode: bit 0 matrix waves, bit 1 vector waves;
// agpr: accumulators in AGPRs (else arch VGPRs); trans: exp2 after each FMA
// (else a second FMA).  Returns the launch's hipError_t.
extern "C" int swa_measure_coexec(float *out, int blocks, int iters_m, int iters_v, int mode,
                                  int agpr, int trans, void *stream) {
    if (!out || blocks < 1 || iters_m < 0 || iters_v < 0) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    const dim3 g(blocks), t(512);
    if (agpr && trans)
        hipLaunchKernelGGL((coexec_kernel<1, 1>), g, t, 0, s, out, iters_m, iters_v, mode);
    else if (agpr)
        hipLaunchKernelGGL((coexec_kernel<1, 0>), g, t, 0, s, out, iters_m, iters_v, mode);
    else if (trans)
        hipLaunchKernelGGL((coexec_kernel<0, 1>), g, t, 0, s, out, iters_m, iters_v, mode);
    else
        hipLaunchKernelGGL((coexec_kernel<0, 0>), g, t, 0, s, out, iters_m, iters_v, mode);
    return (int)hipGetLastError();
}
