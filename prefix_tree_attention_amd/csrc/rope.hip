// Rotary position embedding by tree position ids (AReaL tree-training
// guide, section 打包数据的生成: a token's position id is its ancestor count
// minus one, so a shared prefix is encoded identically in every sequence
// through it).  Half-split rotation of the Qwen/Llama family: with
// f_j = base^(-2j/D) and a_j = pos f_j, the pair (x_j, x_{j+D/2}) is rotated
// by a_j (by -a_j for the inverse, which is also the gradient map).
//
// One lane per (token, pair j) -- or per 16 bytes of pairs when the head
// size allows: the angle and its sine / cosine are formed in float64 (exact
// to float32 rounding at any position), then applied to those pairs of
// every head.  Lanes of one token read and write the two contiguous halves
// of each head vector, so the pass is one coalesced read and write of x:
// HBM-bound.

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

// Same rotation, 16 bytes per access: a lane takes N = 16 / sizeof(T)
// consecutive pairs j0 .. j0 + N - 1 (D / 2 a multiple of N), so each head's
// two halves move as one 16-byte load and store per lane.
template <typename T>
__global__ __launch_bounds__(256) void rope_vec_kernel(const T* x, T* y,  // may alias (in place)
                                                       const int32_t* __restrict__ pos, int64_t L, int H, int D,
                                                       double log2_base, int inverse) {
    constexpr int N = 16 / sizeof(T);
    const int half = D / 2, lanes = half / N;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= L * lanes) return;
    const int64_t i = idx / lanes;
    const int j0 = int(idx % lanes) * N;
    const double p = double(pos[i]);
    float c[N], sn[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        double sd, cd;
        sincos(p * exp2(-2.0 * double(j0 + u) / double(D) * log2_base), &sd, &cd);
        c[u] = float(cd);
        sn[u] = inverse ? -float(sd) : float(sd);
    }
    typedef T vec __attribute__((ext_vector_type(N)));
    auto rot = [&](const vec& a, const vec& b, vec& ya, vec& yb) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const float x1 = to_f(a[u]), x2 = to_f(b[u]);
            ya[u] = from_f<T>(__builtin_fmaf(x1, c[u], -x2 * sn[u]));
            yb[u] = from_f<T>(__builtin_fmaf(x2, c[u], x1 * sn[u]));
        }
    };
    // x and y may be one tensor, so the compiler cannot move a head's loads
    // above the previous head's stores; heads never overlap, so four are
    // loaded explicitly before any of them is stored
    constexpr int kH = 4;
    int h = 0;
    for (; h + kH <= H; h += kH) {
        vec a[kH], b[kH];
#pragma unroll
        for (int u = 0; u < kH; ++u) {
            const int64_t o = (i * H + h + u) * D + j0;
            a[u] = *reinterpret_cast<const vec*>(x + o);
            b[u] = *reinterpret_cast<const vec*>(x + o + half);
        }
#pragma unroll
        for (int u = 0; u < kH; ++u) {
            const int64_t o = (i * H + h + u) * D + j0;
            vec ya, yb;
            rot(a[u], b[u], ya, yb);
            *reinterpret_cast<vec*>(y + o) = ya;
            *reinterpret_cast<vec*>(y + o + half) = yb;
        }
    }
    for (; h < H; ++h) {
        const int64_t o = (i * H + h) * D + j0;
        vec ya, yb;
        rot(*reinterpret_cast<const vec*>(x + o), *reinterpret_cast<const vec*>(x + o + half), ya, yb);
        *reinterpret_cast<vec*>(y + o) = ya;
        *reinterpret_cast<vec*>(y + o + half) = yb;
    }
}

// (cos, sin) of p f_j for every position p < P and pair j < D/2, as the
// rotation passes form them (float64 angle, rounded to float32): the
// operand table of the attention kernels that rotate Q / K where they load
// them and rotate dQ / dK back where they store them.
__global__ __launch_bounds__(256) void rope_table_kernel(float* __restrict__ tab, int64_t P, int D, double log2_base) {
    const int half = D / 2;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= P * half) return;
    const int64_t p = idx / half;
    const int j = int(idx % half);
    double sd, cd;
    sincos(double(p) * exp2(-2.0 * double(j) / double(D) * log2_base), &sd, &cd);
    tab[2 * idx] = float(cd);
    tab[2 * idx + 1] = float(sd);
}

// Rotation of x [L, H, D] bf16 by a (cos, sin) table row per token, eight
// pairs per lane, every head: the K operand of the fused forward.  Same
// arithmetic as the Q rotation inside the forward kernel.
__global__ __launch_bounds__(256) void rope_tab_kernel(const bf16* __restrict__ x, bf16* __restrict__ y,
                                                       const int32_t* __restrict__ pos, const float* __restrict__ tab,
                                                       int64_t L, int H, int D) {
    const int half = D / 2, lanes = half / 8;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= L * lanes) return;
    const int64_t i = idx / lanes;
    const int j0 = int(idx % lanes) * 8;
    const f32x4* t4 = reinterpret_cast<const f32x4*>(tab + (int64_t(pos[i]) * half + j0) * 2);
    const f32x4 c0 = t4[0], c1 = t4[1], c2 = t4[2], c3 = t4[3];
    const float c[8] = {c0[0], c0[2], c1[0], c1[2], c2[0], c2[2], c3[0], c3[2]};
    const float sn[8] = {c0[1], c0[3], c1[1], c1[3], c2[1], c2[3], c3[1], c3[3]};
    for (int h = 0; h < H; ++h) {
        const int64_t o = (i * H + h) * D + j0;
        const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(x + o)), b = __builtin_bit_cast(bf16x8, ld16(x + o + half));
        f32x4 a0, a1, b0, b1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float x1 = float(a[u]), x2 = float(b[u]);
            rope_pair<false>(x1, x2, c[u], sn[u]);
            a0[u] = x1;
            b0[u] = x2;
            float y1 = float(a[u + 4]), y2 = float(b[u + 4]);
            rope_pair<false>(y1, y2, c[u + 4], sn[u + 4]);
            a1[u] = y1;
            b1[u] = y2;
        }
        st16(y + o, __builtin_bit_cast(u32x4, to_bf16x8(a0, a1)));
        st16(y + o + half, __builtin_bit_cast(u32x4, to_bf16x8(b0, b1)));
    }
}

}  // namespace

hipError_t launch_rope_tab(const void* x, void* y, const int32_t* pos, const float* tab, int64_t L, int H, int D,
                           hipStream_t stream) {
    const int64_t n = L * (D / 16);
    if (n <= 0) return hipSuccess;
    rope_tab_kernel<<<unsigned((n + 255) / 256), 256, 0, stream>>>(static_cast<const bf16*>(x), static_cast<bf16*>(y),
                                                                   pos, tab, L, H, D);
    return hipGetLastError();
}

hipError_t launch_rope_table(float* tab, int64_t P, int D, double base, hipStream_t stream) {
    const int64_t n = P * (D / 2);
    if (n <= 0) return hipSuccess;
    rope_table_kernel<<<unsigned((n + 255) / 256), 256, 0, stream>>>(tab, P, D, log2(base));
    return hipGetLastError();
}

hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t L, int H, int D, double base, int inverse,
                       int dtype, hipStream_t stream) {
    const double l2b = log2(base);
    const int elem = dtype == 0 ? 2 : 4, N = 16 / elem;
    const bool vec = (D / 2) % N == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    if (vec) {
        const int64_t n = L * ((D / 2) / N);
        const unsigned grid = unsigned((n + 255) / 256);
        if (dtype == 0)
            rope_vec_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(x), static_cast<bf16*>(y), pos, L,
                                                            H, D, l2b, inverse);
        else
            rope_vec_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), static_cast<float*>(y), pos,
                                                             L, H, D, l2b, inverse);
        return hipGetLastError();
    }
    const int64_t n = L * (D / 2);
    const unsigned grid = unsigned((n + 255) / 256);
    if (dtype == 0)
        rope_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(x), static_cast<bf16*>(y), pos, L, H, D,
                                                    l2b, inverse);
    else
        rope_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), static_cast<float*>(y), pos, L, H,
                                                     D, l2b, inverse);
    return hipGetLastError();
}

}  // namespace treeattn
