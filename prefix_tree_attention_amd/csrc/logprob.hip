// Tree-aware log-probabilities and entropies from the logits of a packed
// batch (AReaL tree-training guide, section "Log Probability 计算：树结构的
// 特殊处理").  A sequence's token k + 1 is predicted by the logits at the
// packed position of its token k; inside a node that is the next position,
// at a node's end it is the row that every child's first token reads.  Every
// packed row is therefore used by all the sequences through it, so the
// row-wise statistics are computed once per packed row (the pages' node
// cache) and the per-sequence values are gathers.
//
//   logits_stats: one workgroup per packed row; a single streaming pass over
//                 the V logits keeps, per lane, a running base-2 reference m
//                 and the sums s, t below (Acc); LSE and entropy follow in
//                 closed form.  HBM-bound: L V elements read once.
//   gather:       one lane per (batch row, column): the prediction of the
//                 row's token j + 1 from the packed position of its token j.

#include <cmath>

#include "device.h"
#include "mfma.h"

namespace treeattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kStatThreads = 256;

// Running per-lane state over a row: base-2 reference m, and with
// a_i = max(x_i log2 e - m, -200) (below -200 the term is 0 in float32):
//   s = sum 2^(a_i),   t = sum 2^(a_i) a_i.
// Then LSE = ln 2 (m + log2 s) and the entropy
//   -sum p ln p = ln 2 (log2 s - t / s)   (p_i = 2^(a_i) / s),
// where m cancels.  A -inf logit gives a_i = -200, a zero term: no NaN.
struct Acc {
    float m, s, t;
};

// rebase (s, t) from reference m to m2 >= m: a_i -> a_i + d, d = m - m2
__device__ __forceinline__ void acc_rebase(Acc& a, float m2) {
    if (a.m == -INFINITY) {
        a.s = a.t = 0.f;
    } else {
        const float d = a.m - m2, f = fast_exp2(d);
        a.t = f * __builtin_fmaf(d, a.s, a.t);
        a.s *= f;
    }
    a.m = m2;
}

__device__ __forceinline__ void acc_merge(Acc& a, Acc b) {
    const float m = fmaxf(a.m, b.m);
    if (m == -INFINITY) return;  // both empty
    acc_rebase(a, m);
    acc_rebase(b, m);
    a.s += b.s;
    a.t += b.t;
}

// fold N values (already in fp32) into the accumulator; one rebase per
// call when their maximum exceeds the running reference
template <int N>
__device__ __forceinline__ void acc_add(Acc& a, const float (&x)[N]) {
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) cm = fmaxf(cm, x[i]);
    cm *= kLog2e;
    if (cm > a.m) acc_rebase(a, cm);
    if (a.m == -INFINITY) return;  // every value so far is -inf: nothing to add
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float ai = fmaxf(__builtin_fmaf(x[i], kLog2e, -a.m), -200.f);
        const float e = fast_exp2(ai);
        a.s += e;
        a.t = __builtin_fmaf(e, ai, a.t);
    }
}

__device__ __forceinline__ float to_f32(bf16 v) { return float(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T>
__global__ __launch_bounds__(kStatThreads) void logits_stats_kernel(const T* __restrict__ logits, int64_t V,
                                                                    float* __restrict__ lse,
                                                                    float* __restrict__ ent) {
    constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte load
    const int64_t row = blockIdx.x;
    const T* __restrict__ p = logits + row * V;
    const int tid = threadIdx.x;
    Acc a{-INFINITY, 0.f, 0.f};
    // scalar head up to 16-byte alignment of the row, vector body, scalar tail
    const int64_t head = int64_t((16 - (reinterpret_cast<uintptr_t>(p) & 15)) & 15) / int64_t(sizeof(T));
    const int64_t h = head < V ? head : V;
    for (int64_t i = tid; i < h; i += kStatThreads) {
        const float x[1] = {to_f32(p[i])};
        acc_add<1>(a, x);
    }
    const int64_t nvec = (V - h) / kVec;
    const u32x4* __restrict__ pv = reinterpret_cast<const u32x4*>(p + h);
    auto fold = [&](const u32x4& w) {
        float x[kVec];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = __uint_as_float(w[j] << 16);
                x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(w[j]);
        }
        acc_add<kVec>(a, x);
    };
    // four 16-byte loads in flight per lane, then their folds
    constexpr int kU = 4;
    int64_t c = tid;
    for (; c + (kU - 1) * kStatThreads < nvec; c += kU * kStatThreads) {
        u32x4 w[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) w[u] = pv[c + u * kStatThreads];
#pragma unroll
        for (int u = 0; u < kU; ++u) fold(w[u]);
    }
    for (; c < nvec; c += kStatThreads) fold(pv[c]);
    for (int64_t i = h + nvec * kVec + tid; i < V; i += kStatThreads) {
        const float x[1] = {to_f32(p[i])};
        acc_add<1>(a, x);
    }
    // workgroup reduction: wave butterfly, then the four waves through LDS
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const Acc b{__shfl_xor(a.m, o), __shfl_xor(a.s, o), __shfl_xor(a.t, o)};
        acc_merge(a, b);
    }
    __shared__ Acc sh[kStatThreads / 64];
    if ((tid & 63) == 0) sh[tid >> 6] = a;
    __syncthreads();
    if (tid == 0) {
        Acc r = sh[0];
#pragma unroll
        for (int w = 1; w < kStatThreads / 64; ++w) acc_merge(r, sh[w]);
        const float l2s = log2f(r.s);
        lse[row] = r.m == -INFINITY ? -INFINITY : kLn2 * (r.m + l2s);
        ent[row] = r.m == -INFINITY ? 0.f : kLn2 * (l2s - r.t / r.s);
    }
}

// `logits` holds the packed rows [row0, row0 + n_rows) of the [L, V] logits;
// entries predicted from a row outside that window are left as they are, so
// windows that cover [0, L) once write every entry once (pads and bad
// positions are written by every call).
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ logits, int64_t row0, int64_t n_rows,
                                                     int64_t L, int64_t V, const float* __restrict__ lse,
                                                     const float* __restrict__ ent, const int32_t* __restrict__ ids,
                                                     const int32_t* __restrict__ row_pos, int64_t B, int64_t S,
                                                     float pad_value, float* __restrict__ out_logp,
                                                     float* __restrict__ out_ent) {
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= B * S) return;
    const int64_t j = e % S;
    // token j of the row predicts token j + 1 (both real when their packed
    // positions are); every index is range-checked, so a bad position or a
    // token id outside the vocabulary gives NaN, never an access out of range
    const int32_t pos = row_pos[e];
    const int32_t nxt = j + 1 < S ? row_pos[e + 1] : -1;
    float lp = pad_value, en = pad_value;
    if (pos >= 0 && nxt >= 0) {
        if (pos < L && nxt < L) {
            if (pos < row0 || pos >= row0 + n_rows) return;
            const int32_t label = ids[nxt];
            lp = (label >= 0 && label < V) ? to_f32(logits[(pos - row0) * V + label]) - lse[pos] : NAN;
            en = ent[pos];
        } else {
            lp = en = NAN;
        }
    }
    out_logp[e] = lp;
    out_ent[e] = en;
}

}  // namespace

hipError_t launch_logits_stats(const void* logits, int64_t L, int64_t V, int dtype, float* lse, float* ent,
                               hipStream_t stream) {
    if (dtype == 0)
        logits_stats_kernel<bf16><<<unsigned(L), kStatThreads, 0, stream>>>(static_cast<const bf16*>(logits), V, lse,
                                                                            ent);
    else
        logits_stats_kernel<float><<<unsigned(L), kStatThreads, 0, stream>>>(static_cast<const float*>(logits), V,
                                                                             lse, ent);
    return hipGetLastError();
}

hipError_t launch_gather_logprobs(const void* logits, int64_t row0, int64_t n_rows, int64_t L, int64_t V, int dtype,
                                  const float* lse, const float* ent, const int32_t* ids, const int32_t* row_pos,
                                  int64_t B, int64_t S, float pad_value, float* out_logp, float* out_ent,
                                  hipStream_t stream) {
    const int64_t n = B * S;
    const unsigned grid = unsigned((n + 255) / 256);
    if (dtype == 0)
        gather_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(logits), row0, n_rows, L, V, lse, ent,
                                                      ids, row_pos, B, S, pad_value, out_logp, out_ent);
    else
        gather_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(logits), row0, n_rows, L, V, lse,
                                                       ent, ids, row_pos, B, S, pad_value, out_logp, out_ent);
    return hipGetLastError();
}

}  // namespace treeattn
