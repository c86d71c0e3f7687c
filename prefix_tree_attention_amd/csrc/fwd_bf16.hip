// Forward tree attention, bf16 in / fp32 accumulate, gfx950 MFMA.
//
// What it computes (AReaL tree-training guide, packing figure: a token
// attends to itself and its ancestors only; key j is visible to query i iff
// j <= i <= se[j] in the pre-order layout):
//   O_i = sum_{j in A(i)} softmax_j(scale q_i.k_j) v_j,
//   LSE_i = ln sum_{j in A(i)} exp(scale q_i.k_j).
//
// Work decomposition: one workgroup (4 waves) per (128-query block, query
// head); wave w owns queries 32w..32w+31 of the block as two 16-column MFMA
// groups.  The workgroup walks only the nonempty key tiles of its query
// block (row list of the metadata), 64 keys per pipeline step.  K and V of a
// step go HBM -> LDS by direct loads into double-buffered swizzled tiles
// (tile.h) while the previous step computes.  Partial tiles apply the
// subtree-interval predicate; full tiles skip it.
//
// Products are computed transposed: S^T = K Q^T (A = K rows from LDS, B =
// Q^T held in registers), O^T = V^T P^T (A = V^T read from the row-major V
// tile by transposing LDS loads, B = P^T taken straight from the S^T
// accumulators).  Each lane thus owns one query column, so softmax
// statistics need only an in-lane reduction plus two cross-lane steps, and
// the rescaling of O^T is per lane.  S^T block b covers keys 16b..16b+15;
// k-step c of the PV product pairs blocks 2c and 2c+1, and the transposing
// reads of V take exactly the key rows those accumulator lanes hold.
// Softmax runs in base 2 with scale*log2(e) folded into one FMA.

#include <cmath>

#include "device.h"
#include "mfma.h"
#include "tile.h"

namespace treeattn {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = kTileRows;  // keys per pipeline step
constexpr float kRescaleSlack = 8.f;  // log2 units: p <= 256 between rescales

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ se,
    const int32_t* __restrict__ q_order, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ row_ent, int L, int Hq, int Hkv, float scale_log2) {
    using T = Tile<D>;
    constexpr int NS = D / 32;  // k-steps of QK^T
    constexpr int NT = D / 16;  // d-blocks of O^T
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * T::kBytes];
    lds_char* const smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    // work item: key/value-head major, then query blocks heaviest first,
    // then the query heads of the group
    const int G = Hq / Hkv, per_kv = (int(gridDim.x) / Hq) * G;
    const int work = xcd_logical_block();
    const int hkv = work / per_kv, rank = (work % per_kv) / G, h = hkv * G + work % G;
    const int qb = q_order[rank];
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int qrow0 = qb * kBlock + 32 * wave;  // first query of this wave

    // Q^T operand: lane holds query (qrow0 + 16 qs + n), d = 32 s + 8 g .. +7
    bf16x8 qf[2][NS];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qf[qs][s] = __builtin_bit_cast(
                bf16x8, ld16(Q + int64_t(qrow0 + 16 * qs + n) * q_stride + int64_t(h) * D + 32 * s + 8 * g));

    f32x4 oacc[2][NT];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < NT; ++t) oacc[qs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    const int beg = row_ptr[qb], nsteps = 2 * (row_ptr[qb + 1] - beg);
    const int kvs = int(kv_stride);
    auto ktile = [&](int buf) { return smem + (2 * buf) * T::kBytes; };
    auto vtile = [&](int buf) { return smem + (2 * buf + 1) * T::kBytes; };
    auto issue = [&](int st, int buf) {
        const int kbase = (row_ent[beg + (st >> 1)] >> 1) * kBlock + kStep * (st & 1);
        const int64_t off = int64_t(kbase) * kv_stride + int64_t(hkv) * D;
        T::load_async(ktile(buf), K + off, kvs, wave, lane);
        T::load_async(vtile(buf), V + off, kvs, wave, lane);
    };
    if (nsteps > 0) issue(0, 0);
    wait_vm_all();
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int ent = row_ent[beg + (st >> 1)];
        const int kbase = (ent >> 1) * kBlock + kStep * (st & 1);
        const bool partial = ent & 1;
        if (st + 1 < nsteps) issue(st + 1, buf ^ 1);
        const lds_char* kt = ktile(buf);
        const lds_char* vt = vtile(buf);

        // S^T = K Q^T (unscaled): block b = keys 16b..16b+15; lane holds
        // query column n of group qs, keys 16b + 4g + 0..3
        f32x4 sc[2][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bf16x8 a[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) a[s] = T::row_frag(kt, 16 * b + n, 4 * s + g);
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s) c = mfma16x16x32(a[s], qf[qs][s], c);
                sc[qs][b] = c;
            }
        }

        if (partial) {
            i32x4 sek[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) sek[b] = *reinterpret_cast<const i32x4*>(se + kbase + 16 * b + 4 * g);
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                const int qi = qrow0 + 16 * qs + n;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kbase + 16 * b + 4 * g + r;
                        if (!(key <= qi && qi <= sek[b][r])) sc[qs][b][r] = -INFINITY;
                    }
            }
        }

        // online softmax in base 2, one query column per lane; the running
        // max is kept in scaled units and the scale is folded into the FMA
        // that forms the exp2 argument.
        bf16x8 pb[2][2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            // maximum (not maxnum) chains lower to v_maximum3_f32 with no
            // NaN-quieting of the accumulator inputs
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[qs][b][0]), sc[qs][b][1]);
                mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[qs][b][2]), sc[qs][b][3]);
            }
            mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16));
            mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32));
            // The reference max only moves when some lane's tile max exceeds
            // it by more than kRescaleSlack (log2 units).  O and l are both
            // relative to the same reference, so a stale one changes nothing
            // but the magnitude of p, which stays <= 2^kRescaleSlack; the
            // O rescale thus runs a few times per row instead of nearly
            // every step.
            const float mt = mx * scale_log2;
            if (__any(mt > m_run[qs] + kRescaleSlack)) {
                const float mnew = fmaxf(m_run[qs], mt);
                const float alpha = fast_exp2(m_run[qs] - (mnew == -INFINITY ? 0.f : mnew));
                l_run[qs] *= alpha;
#pragma unroll
                for (int t = 0; t < NT; ++t) oacc[qs][t] *= alpha;
                m_run[qs] = mnew;
            }
            const float muse = m_run[qs] == -INFINITY ? 0.f : m_run[qs];
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(sc[qs][b][r], scale_log2, -muse));
                    sc[qs][b][r] = p;
                    rs += p;
                }
            l_run[qs] += rs;
            pb[qs][0] = to_bf16x8(sc[qs][0], sc[qs][1]);
            pb[qs][1] = to_bf16x8(sc[qs][2], sc[qs][3]);
        }

        // O^T += V^T P^T: k-step c pairs key rows 32c + 4g + 0..3 and
        // 32c + 16 + 4g + 0..3 (blocks 2c and 2c+1)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 a = join_tr(T::tr_frag(vt, 32 * c + 4 * g, 16 * t, n),
                                         T::tr_frag(vt, 32 * c + 16 + 4 * g, 16 * t, n));
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) oacc[qs][t] = mfma16x16x32(a, pb[qs][c], oacc[qs][t]);
            }

        wait_vm_all();
        __syncthreads();
    }

    // epilogue: normalise, write O (bf16) and LSE (natural log)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        float l = l_run[qs];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int qi = qrow0 + 16 * qs + n;
        bf16* orow = O + int64_t(qi) * q_stride + int64_t(h) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 v = oacc[qs][t] * inv;
            st8(orow + 16 * t + 4 * g, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
        }
        if (g == 0) LSE[int64_t(h) * L + qi] = l > 0.f ? (m_run[qs] + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int32_t* se, const MetaPtrs& mp, const AttnShape& sh,
                           hipStream_t stream) {
    const dim3 grid(unsigned(sh.nb) * unsigned(sh.Hq));
    const float sl2 = sh.scale * 1.4426950408889634f;
    const auto* Q = static_cast<const bf16*>(q);
    const auto* K = static_cast<const bf16*>(k);
    const auto* V = static_cast<const bf16*>(v);
    auto* O = static_cast<bf16*>(o);
    if (sh.D == 128)
        fwd_bf16_kernel<128><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, mp.q_order, mp.row_ptr,
                                                             mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2);
    else if (sh.D == 64)
        fwd_bf16_kernel<64><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, mp.q_order, mp.row_ptr,
                                                            mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace treeattn
