// Device helpers of the depth-first (DTA) execution: the subtree ends of a
// stack frame, row copies between the packed layout and the frame, and the
// float32 gradient accumulators' conversion.  All HBM-bound and small; the
// attention itself runs in the tree kernels over the frame.

#include "device.h"
#include "mfma.h"

namespace treeattn {
namespace {

constexpr int kThreadsDfs = 256;

// Subtree ends of a frame: a stack segment's rows reach the frame's last real
// row (every stack key is an ancestor of every later real token); the leaf
// rows being run take the packed layout's subtree ends, shifted; the rest
// (padding between and after segments) is -1.
__global__ __launch_bounds__(kThreadsDfs) void dfs_se_kernel(int32_t* __restrict__ se, int64_t rows,
                                                             const int32_t* __restrict__ packed_se,
                                                             DfsSegments a) {
    const int64_t i = int64_t(blockIdx.x) * kThreadsDfs + threadIdx.x;
    if (i >= rows) return;
    int v = -1;
    for (int s = 0; s < a.n; ++s)
        if (i >= a.row0[s] && i < a.row0[s] + a.len[s]) v = a.top_se;
    if (i >= a.leaf_row0 && i < a.leaf_row0 + a.leaf_len) {
        const int32_t p = packed_se[a.leaf_p0 + (i - a.leaf_row0)];
        v = p - a.leaf_p0 + a.leaf_row0;
    }
    se[i] = v;
}

// nrows rows of row_bytes (a multiple of 16) from src row s0 to dst row d0
__global__ __launch_bounds__(kThreadsDfs) void dfs_copy_rows_kernel(const char* __restrict__ src,
                                                                    char* __restrict__ dst, int64_t s0, int64_t d0,
                                                                    int64_t nrows, int64_t row_bytes) {
    const int64_t per = row_bytes / 16;
    const int64_t n = nrows * per;
    for (int64_t c = int64_t(blockIdx.x) * kThreadsDfs + threadIdx.x; c < n;
         c += int64_t(gridDim.x) * kThreadsDfs) {
        const int64_t r = c / per, w = c % per;
        st16(dst + (d0 + r) * row_bytes + 16 * w, ld16(src + (s0 + r) * row_bytes + 16 * w));
    }
}

// per head h < H: dst[h * Ld + d0 + i] = src[h * Ls + s0 + i], i < n
__global__ __launch_bounds__(kThreadsDfs) void dfs_copy_cols_kernel(const float* __restrict__ src,
                                                                    float* __restrict__ dst, int64_t Ls, int64_t Ld,
                                                                    int64_t s0, int64_t d0, int64_t n, int H) {
    const int64_t total = n * H;
    for (int64_t c = int64_t(blockIdx.x) * kThreadsDfs + threadIdx.x; c < total;
         c += int64_t(gridDim.x) * kThreadsDfs) {
        const int64_t h = c / n, i = c % n;
        dst[h * Ld + d0 + i] = src[h * Ls + s0 + i];
    }
}

// fill n 16-byte words with a 32-bit pattern
__global__ __launch_bounds__(kThreadsDfs) void dfs_fill_kernel(char* __restrict__ p, int64_t n16, uint32_t pat) {
    const u32x4 v = {pat, pat, pat, pat};
    for (int64_t c = int64_t(blockIdx.x) * kThreadsDfs + threadIdx.x; c < n16;
         c += int64_t(gridDim.x) * kThreadsDfs)
        st16(p + 16 * c, v);
}

// per head h < H: p[h * L + i] = value for i in [i0, i0 + n)
__global__ __launch_bounds__(kThreadsDfs) void dfs_fill_cols_kernel(float* __restrict__ p, int64_t L, int64_t i0,
                                                                    int64_t n, int H, float value) {
    const int64_t total = n * H;
    for (int64_t c = int64_t(blockIdx.x) * kThreadsDfs + threadIdx.x; c < total;
         c += int64_t(gridDim.x) * kThreadsDfs)
        p[(c / n) * L + i0 + c % n] = value;
}

// float32 accumulator rows [s0, s0 + nrows) x width -> bf16 rows from d0
__global__ __launch_bounds__(kThreadsDfs) void dfs_emit_kernel(const float* __restrict__ acc, bf16* __restrict__ out,
                                                               int64_t s0, int64_t d0, int64_t nrows, int64_t width) {
    const int64_t per = width / 8;
    const int64_t n = nrows * per;
    for (int64_t c = int64_t(blockIdx.x) * kThreadsDfs + threadIdx.x; c < n;
         c += int64_t(gridDim.x) * kThreadsDfs) {
        const int64_t r = c / per, w = c % per;
        const f32x4* a = reinterpret_cast<const f32x4*>(acc + (s0 + r) * width + 8 * w);
        const f32x4 x = a[0], y = a[1];
        st16(out + (d0 + r) * width + 8 * w,
             u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])});
    }
}

// p[i] = i, i < n (query-block lists)
__global__ __launch_bounds__(kThreadsDfs) void dfs_iota_kernel(int32_t* __restrict__ p, int n) {
    const int i = int(blockIdx.x) * kThreadsDfs + int(threadIdx.x);
    if (i < n) p[i] = i;
}

unsigned grid_for(int64_t work) {
    const int64_t b = (work + kThreadsDfs - 1) / kThreadsDfs;
    return unsigned(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

}  // namespace

hipError_t launch_dfs_se(int32_t* se, int64_t rows, const int32_t* packed_se, const DfsSegments& a,
                         hipStream_t stream) {
    dfs_se_kernel<<<unsigned((rows + kThreadsDfs - 1) / kThreadsDfs), kThreadsDfs, 0, stream>>>(se, rows, packed_se,
                                                                                               a);
    return hipGetLastError();
}

hipError_t launch_dfs_copy_rows(const void* src, void* dst, int64_t s0, int64_t d0, int64_t nrows, int64_t row_bytes,
                                hipStream_t stream) {
    if (nrows <= 0) return hipSuccess;
    dfs_copy_rows_kernel<<<grid_for(nrows * row_bytes / 16), kThreadsDfs, 0, stream>>>(
        static_cast<const char*>(src), static_cast<char*>(dst), s0, d0, nrows, row_bytes);
    return hipGetLastError();
}

hipError_t launch_dfs_copy_cols(const float* src, float* dst, int64_t Ls, int64_t Ld, int64_t s0, int64_t d0,
                                int64_t n, int H, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    dfs_copy_cols_kernel<<<grid_for(n * H), kThreadsDfs, 0, stream>>>(src, dst, Ls, Ld, s0, d0, n, H);
    return hipGetLastError();
}

hipError_t launch_dfs_fill(void* p, int64_t bytes, uint32_t pattern, hipStream_t stream) {
    if (bytes <= 0) return hipSuccess;
    dfs_fill_kernel<<<grid_for(bytes / 16), kThreadsDfs, 0, stream>>>(static_cast<char*>(p), bytes / 16, pattern);
    return hipGetLastError();
}

hipError_t launch_dfs_fill_cols(float* p, int64_t L, int64_t i0, int64_t n, int H, float value, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    dfs_fill_cols_kernel<<<grid_for(n * H), kThreadsDfs, 0, stream>>>(p, L, i0, n, H, value);
    return hipGetLastError();
}

hipError_t launch_dfs_iota(int32_t* p, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    dfs_iota_kernel<<<unsigned((n + kThreadsDfs - 1) / kThreadsDfs), kThreadsDfs, 0, stream>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_dfs_emit(const float* acc, void* out, int64_t s0, int64_t d0, int64_t nrows, int64_t width,
                           hipStream_t stream) {
    if (nrows <= 0) return hipSuccess;
    dfs_emit_kernel<<<grid_for(nrows * width / 8), kThreadsDfs, 0, stream>>>(acc, static_cast<bf16*>(out), s0, d0,
                                                                            nrows, width);
    return hipGetLastError();
}

}  // namespace treeattn
