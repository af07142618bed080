// probe.hip -- self-check of the matrix-core fragment abstraction.
#include "clr_kernels.h"

namespace clr {

// One wave: C = A * Bt^T, A and Bt 16 x 32 row-major.  Also exercises the
// accumulator -> B-fragment chaining: C2 = A[:, :16|16:32] chained through
// an identity product, written to C + 256.
template <typename E>
__global__ __launch_bounds__(64) void probe_mma_kernel(const E* A, const E* Bt, float* C) {
    const int l = threadIdx.x, r = l & 15, g = l >> 4;
    Frag<E> fa = ldfrag(A + r * 32 + 4 * g);
    Frag<E> fb = ldfrag(Bt + r * 32 + 4 * g);
    f32x4 acc = zero4();
    mma(acc, fa, fb);
#pragma unroll
    for (int i = 0; i < 4; ++i) C[(4 * g + i) * 16 + r] = acc[i];
    // chaining: D1 = Bt[:, 0:16]^T as accumulator tiles via identity product,
    // then C2 = A * (rows of D1 and D2 as B fragment) must equal C.
    // Build the two accumulator tiles holding B[k][n] = Bt[n][k] for k in
    // 0..15 and 16..31 directly from memory in accumulator layout.
    f32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = to_f(Bt[r * 32 + 4 * g + i]);
        hi[i] = to_f(Bt[r * 32 + 16 + 4 * g + i]);
    }
    Frag<E> fb2 = frag_from_acc<E>(lo, hi);
    f32x4 acc2 = zero4();
    mma(acc2, fa, fb2);
#pragma unroll
    for (int i = 0; i < 4; ++i) C[256 + (4 * g + i) * 16 + r] = acc2[i];
}

hipError_t launch_probe_mma(int bf16_, const void* A, const void* Bt, float* C, hipStream_t st) {
    if (bf16_)
        hipLaunchKernelGGL(probe_mma_kernel<bf16>, dim3(1), dim3(64), 0, st, (const bf16*)A, (const bf16*)Bt, C);
    else
        hipLaunchKernelGGL(probe_mma_kernel<float>, dim3(1), dim3(64), 0, st, (const float*)A, (const float*)Bt, C);
    return hipGetLastError();
}

}  // namespace clr
