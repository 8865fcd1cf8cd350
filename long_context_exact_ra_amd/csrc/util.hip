// util.hip -- running-state initialisation and the final rescale.
//
// Final rescale (slowleelab "Ring Attention" page, 4.3: the output is divided by
// the running sum once, after the last block): O_acc[row, :] /= l[row], with an
// optional copy in the input dtype (bf16 rounded to nearest even).
// Initial state: O_acc = 0, m = -inf, l = 0; merging one block into it yields
// that block's own attention.  Written with plain stores (no memset nodes), so
// the call can be captured in a HIP graph.
#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void init_kernel(float *O_acc, float *m, float *l,
                                                   int64_t rows, int d) {
    const int64_t n4 = rows * d / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        ((f32x4 *)O_acc)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) {
        m[i] = -INFINITY;
        l[i] = 0.f;
    }
}

// One thread per 4 consecutive elements of a row (d is a multiple of 4).
__global__ __launch_bounds__(256) void finalize_kernel(float *O_acc, const float *l,
                                                       int64_t rows, int d, int dtype,
                                                       void *O_out) {
    const int64_t n4 = rows * d / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const int64_t row = (i * 4) / d;
        const float den = l[row];
        f32x4 v = ((f32x4 *)O_acc)[i];
        v = f32x4{v[0] / den, v[1] / den, v[2] / den, v[3] / den};
        ((f32x4 *)O_acc)[i] = v;
        if (O_out) {
            if (dtype == 1)
                ((bf16x4 *)O_out)[i] = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2],
                                              (__bf16)v[3]};
            else
                ((f32x4 *)O_out)[i] = v;
        }
    }
}

int grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (int)g;
}

}  // namespace

hipError_t launch_state_init(float *O_acc, float *m, float *l, int64_t rows, int d,
                             hipStream_t st) {
    const int64_t n = rows * d / 4 > rows ? rows * d / 4 : rows;
    hipLaunchKernelGGL(init_kernel, dim3(grid_for(n)), dim3(256), 0, st, O_acc, m, l, rows, d);
    return hipGetLastError();
}

hipError_t launch_finalize(float *O_acc, const float *l, int64_t rows, int d, int dtype,
                           void *O_out, hipStream_t st) {
    hipLaunchKernelGGL(finalize_kernel, dim3(grid_for(rows * d / 4)), dim3(256), 0, st, O_acc,
                       l, rows, d, dtype, O_out);
    return hipGetLastError();
}

}  // namespace ra
