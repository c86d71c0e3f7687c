// Rotary position embedding by tree position ids (AReaL tree-training
// guide, section 打包数据的生成: a token's position id is its ancestor count
// minus one, so a shared prefix is encoded identically in every sequence
// through it).  Half-split rotation of the Qwen/Llama family: with
// f_j = base^(-2j/D) and a_j = pos f_j, the pair (x_j, x_{j+D/2}) is rotated
// by a_j (by -a_j for the inverse, which is also the gradient map).
//
// One lane per (token, pair j): the angle and its sine / cosine are formed
// in float64 (exact to float32 rounding at any position), then applied to
// that pair of every head.  Lanes of one token read and write the two
// contiguous halves of each head vector, so the pass is one coalesced read
// and write of x: HBM-bound.

#include "device.h"
#include "mfma.h"

namespace treeattn {
namespace {

__device__ __forceinline__ float to_f(bf16 v) { return float(v); }
__device__ __forceinline__ float to_f(float v) { return v; }
template <typename T>
__device__ __forceinline__ T from_f(float v) {
    return T(v);
}

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(const T* x, T* y,  // may alias (in place)
                                                   const int32_t* __restrict__ pos, int64_t L, int H, int D,
                                                   double log2_base, int inverse) {
    const int half = D / 2;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= L * half) return;
    const int64_t i = idx / half;
    const int j = int(idx % half);
    const double ang = double(pos[i]) * exp2(-2.0 * double(j) / double(D) * log2_base);
    double sd, cd;
    sincos(ang, &sd, &cd);
    const float c = float(cd), s = inverse ? -float(sd) : float(sd);
    for (int h = 0; h < H; ++h) {
        const int64_t o = (i * H + h) * D + j;
        const float x1 = to_f(x[o]), x2 = to_f(x[o + half]);
        y[o] = from_f<T>(__builtin_fmaf(x1, c, -x2 * s));
        y[o + half] = from_f<T>(__builtin_fmaf(x2, c, x1 * s));
    }
}

}  // namespace

hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t L, int H, int D, double base, int inverse,
                       int dtype, hipStream_t stream) {
    const int64_t n = L * (D / 2);
    const unsigned grid = unsigned((n + 255) / 256);
    const double l2b = log2(base);
    if (dtype == 0)
        rope_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(x), static_cast<bf16*>(y), pos, L, H, D,
                                                    l2b, inverse);
    else
        rope_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), static_cast<float*>(y), pos, L, H,
                                                     D, l2b, inverse);
    return hipGetLastError();
}

}  // namespace treeattn
