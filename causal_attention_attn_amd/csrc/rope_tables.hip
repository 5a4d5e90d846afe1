// RoPE cosine/sine tables: cos_tab[t][i] = cos(t * theta_i), sin_tab[t][i] =
// sin(t * theta_i), theta_i = base^(-2i/D). Rotary position embedding on the
// query/key projections is what the pages use to encode relative positions
// ("Tiny Hackable CUDA", section 3). The angle and its cosine/sine are evaluated
// in double precision (an fp32 angle would be off by up to ~5e-4 rad at
// t = 8191) and rounded once to fp32.
#include <hip/hip_runtime.h>

#include "launchers.h"

namespace attn {

__global__ void rope_tables_kernel(float* __restrict__ cs, float* __restrict__ sn, int T,
                                   int half, int D, double base) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)T * half) return;
    const int t = (int)(idx / half), i = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)i / (double)D);
    double s, c;
    sincos((double)t * theta, &s, &c);
    cs[idx] = (float)c;
    sn[idx] = (float)s;
}

hipError_t launch_rope_tables(float* cs, float* sn, int T, int D, double base, hipStream_t st) {
    const long n = (long)T * (D / 2);
    const int threads = 256;
    const long blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, cs, sn,
                       T, D / 2, D, base);
    return hipGetLastError();
}

}  // namespace attn
