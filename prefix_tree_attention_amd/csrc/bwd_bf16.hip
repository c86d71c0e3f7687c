// Backward tree attention, bf16 in / fp32 accumulate, gfx950 MFMA.
//
// With P = softmax of the visible scores (recomputed from LSE) and
// Delta_i = dO_i . O_i:
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - Delta_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i,
// summed, for dK / dV, over the query heads sharing a key/value head.  A
// shared prefix token is a single key column, so its gradient is the sum
// over every sequence below it (AREAL-DTA notes, §3 问题形式化) with no
// extra work.
//
// Three kernels:
//   delta: Delta for every (token, query head).
//   dkdv:  one workgroup per (128-key block, key/value head); wave w owns
//          keys 32w..32w+31 and keeps K^T, V^T operands and the dK^T, dV^T
//          accumulators in registers.  It walks the nonempty tiles of its
//          key block (column list) for each query head of the group, 64
//          queries per step; Q and dO (and LSE, Delta) of a step go HBM ->
//          LDS by direct loads into double-buffered swizzled tiles.
//            S = Q K^T, dP = dO V^T      (A = Q / dO rows of the tiles)
//            dV^T += dO^T P, dK^T += Q^T dS
//          (A = dO^T / Q^T by transposing LDS reads of the same tiles,
//          B = P / dS straight from the score accumulators).
//   dq:    one workgroup per (128-query block, query head) like the forward:
//            S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T,
//          K^T again by transposing reads of the K tile.
// Score block b of a 64-row step covers rows 16b..16b+15; the gradient
// products' k-step c pairs blocks 2c and 2c+1, whose accumulator lanes hold
// rows 32c + 4g + 0..3 and 32c + 16 + 4g + 0..3 -- exactly the rows the
// transposing reads fetch.

#include <cmath>
#include <type_traits>

#include "device.h"
#include "mfma.h"
#include "tile.h"

namespace treeattn {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = kTileRows;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O), and LSE in base 2 (LSE log2 e) for the dK/dV
// kernel's exponent
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_bf16_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                         const float* __restrict__ LSE, float* __restrict__ delta,
                                                         float* __restrict__ lse2, int L, int Hq) {
    const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (r >= int64_t(L) * Hq) return;
    const int64_t hr = int64_t(r % Hq) * L + r / Hq;
    lse2[hr] = LSE[hr] * kLog2e;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        const u32x4 a = ld16(O + r * D + 8 * c), b = ld16(dO + r * D + 8 * c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc += bf16_to_float(a[w] & 0xffffu) * bf16_to_float(b[w] & 0xffffu);
            acc += bf16_to_float(a[w] >> 16) * bf16_to_float(b[w] >> 16);
        }
    }
    delta[hr] = acc;
}

// Place a value in accumulation registers (empty asm with an AGPR operand).
__device__ __forceinline__ void pin_agpr(bf16x8& x) {
    i32x4 v = __builtin_bit_cast(i32x4, x);
    asm volatile("" : "+a"(v));
    x = __builtin_bit_cast(bf16x8, v);
}

// direct load of 64 consecutive floats (one wave)
__device__ __forceinline__ void load_row64_async(lds_char* dst, const float* __restrict__ src, int lane) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + lane), reinterpret_cast<lds_void*>(dst), 4, 0,
                                     0);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, const int32_t* __restrict__ se,
    const int32_t* __restrict__ k_order, const int32_t* __restrict__ col_ptr,
    const int32_t* __restrict__ col_ent, int L, int Hq, int Hkv, float scale_log2, float scale) {
    using T = Tile<D>;
    constexpr int NS = D / 32, NT = D / 16;
    constexpr int kStage = 2 * T::kBytes + 512;  // Q tile, dO tile, LSE log2 e [64], Delta[64]
    __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kStage];
    lds_char* const smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    // work item: key/value-head major, then key blocks heaviest first
    const int nbk = int(gridDim.x) / Hkv;
    const int work = xcd_logical_block();
    const int hkv = work / nbk, rank = work % nbk;
    const int kb = k_order[rank];
    const int G = Hq / Hkv;
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int kw0 = kb * kBlock + 32 * wave;

    // K^T, V^T operands of this wave's 32 keys: lane holds key (kw0 + 16 ks + n)
    bf16x8 kf[2][NS], vf[2][NS];
    int sek[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int key = kw0 + 16 * ks + n;
        sek[ks] = se[key];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kf[ks][s] = __builtin_bit_cast(bf16x8, ld16(K + int64_t(key) * kv_stride + hkv * D + 32 * s + 8 * g));
            vf[ks][s] = __builtin_bit_cast(bf16x8, ld16(V + int64_t(key) * kv_stride + hkv * D + 32 * s + 8 * g));
        }
    }
    // The resident K/V operands live in the accumulation-register file: MFMA
    // reads its A/B operands from either file, and the vector registers are
    // needed for the dK/dV accumulators and the per-step scores.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            pin_agpr(kf[ks][s]);
            pin_agpr(vf[ks][s]);
        }
    f32x4 dk[2][NT], dv[2][NT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int t = 0; t < NT; ++t) dk[ks][t] = dv[ks][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the column is walked from its last query block down, so the key blocks
    // in flight on an XCD read the same Q / dO tiles at about the same time
    const int beg = col_ptr[kb], nsteps = (col_ptr[kb + 1] - beg) * 2 * G;
    const int last = col_ptr[kb + 1] - 1;
    const int qs32 = int(q_stride);
    auto qtile = [&](int buf) { return smem + buf * kStage; };
    auto gtile = [&](int buf) { return smem + buf * kStage + T::kBytes; };
    auto lsev = [&](int buf) { return smem + buf * kStage + 2 * T::kBytes; };
    auto dlv = [&](int buf) { return smem + buf * kStage + 2 * T::kBytes + 256; };
    // Steps run over the query heads of the group fastest, then the two
    // 64-query halves of a tile, then the tiles col_ent[last], col_ent[last-1],
    // ...; the position is kept as counters (tile, half, head) so the loop
    // carries no integer division.
    struct StepPos {
        int tile, half, head;
    };
    auto advance = [&](StepPos& p) {
        if (++p.head == G) {
            p.head = 0;
            if (++p.half == 2) {
                p.half = 0;
                ++p.tile;
            }
        }
    };
    auto issue = [&](const StepPos& p, int buf) {
        const int ent = col_ent[last - p.tile];
        const int qbase = (ent >> 1) * kBlock + kStep * p.half;
        const int h = hkv * G + p.head;
        const int64_t off = int64_t(qbase) * q_stride + int64_t(h) * D;
        T::load_async(qtile(buf), Q + off, qs32, wave, lane);
        T::load_async(gtile(buf), dO + off, qs32, wave, lane);
        if (wave == 0) load_row64_async(lsev(buf), LSE2 + int64_t(h) * L + qbase, lane);
        if (wave == 1) load_row64_async(dlv(buf), Delta + int64_t(h) * L + qbase, lane);
    };
    StepPos cur{0, 0, 0}, nxt{0, 0, 0};
    if (nsteps > 0) {
        issue(nxt, 0);
        advance(nxt);
    }
    wait_vm_all();
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int ent = col_ent[last - cur.tile];
        const int qbase = (ent >> 1) * kBlock + kStep * cur.half;
        const bool partial = ent & 1;
        advance(cur);
        if (st + 1 < nsteps) {
            issue(nxt, buf ^ 1);
            advance(nxt);
        }
        const lds_char* qt = qtile(buf);
        const lds_char* gt = gtile(buf);
        const lds_char* lsp = lsev(buf);
        const lds_char* dlp = dlv(buf);

        // two halves of 32 queries: blocks b = 2c, 2c+1 feed k-step c of the
        // gradient products
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // dP accumulates onto -Delta, so it leaves the products as dP - Delta
            f32x4 ndl[2];
#pragma unroll
            for (int e = 0; e < 2; ++e)
                ndl[e] = -*reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                    dlp + 4 * (32 * c + 16 * e + 4 * g));
            f32x4 s[2][2], dp[2][2];  // [ks][e]: lane = key column, queries 32c + 16e + 4g + 0..3
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int b = 2 * c + e;
                bf16x8 aq[NS], ag[NS];
#pragma unroll
                for (int x = 0; x < NS; ++x) {
                    aq[x] = T::row_frag(qt, 16 * b + n, 4 * x + g);
                    ag[x] = T::row_frag(gt, 16 * b + n, 4 * x + g);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    f32x4 cs = {0.f, 0.f, 0.f, 0.f}, cd = ndl[e];
#pragma unroll
                    for (int x = 0; x < NS; ++x) {
                        cs = mfma16x16x32(aq[x], kf[ks][x], cs);
                        cd = mfma16x16x32(ag[x], vf[ks][x], cd);
                    }
                    s[ks][e] = cs;
                    dp[ks][e] = cd;
                }
            }
            f32x4 l2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e)
                l2[e] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                    lsp + 4 * (32 * c + 16 * e + 4 * g));
            bf16x8 pb[2], db[2];
            // P = exp2(scale log2e S - LSE log2e), dS = P (dP - Delta); the
            // subtree-interval predicate only in partial tiles (separate code
            // path so full tiles carry no mask arithmetic)
            auto elementwise = [&](auto masked) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int key = kw0 + 16 * ks + n;
#pragma unroll
                    for (int e = 0; e < 2; ++e)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float p = fast_exp2(__builtin_fmaf(s[ks][e][r], scale_log2, -l2[e][r]));
                            if constexpr (decltype(masked)::value) {
                                const int qi = qbase + 32 * c + 16 * e + 4 * g + r;
                                p = (key <= qi && qi <= sek[ks]) ? p : 0.f;
                            }
                            s[ks][e][r] = p;
                            dp[ks][e][r] = p * dp[ks][e][r];
                        }
                    pb[ks] = to_bf16x8(s[ks][0], s[ks][1]);
                    db[ks] = to_bf16x8(dp[ks][0], dp[ks][1]);
                }
            };
            if (partial)
                elementwise(std::true_type{});
            else
                elementwise(std::false_type{});
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 ag = join_tr(T::tr_frag(gt, 32 * c + 4 * g, 16 * t, n),
                                          T::tr_frag(gt, 32 * c + 16 + 4 * g, 16 * t, n));
                const bf16x8 aq = join_tr(T::tr_frag(qt, 32 * c + 4 * g, 16 * t, n),
                                          T::tr_frag(qt, 32 * c + 16 + 4 * g, 16 * t, n));
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    dv[ks][t] = mfma16x16x32(ag, pb[ks], dv[ks][t]);
                    dk[ks][t] = mfma16x16x32(aq, db[ks], dk[ks][t]);
                }
            }
        }

        wait_vm_all();
        __syncthreads();
    }

    // lane holds key (kw0 + 16 ks + n), d = 16 t + 4 g .. +3
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int64_t off = int64_t(kw0 + 16 * ks + n) * kv_stride + hkv * D + 4 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 a = dk[ks][t] * scale, b = dv[ks][t];
            st8(dK + off + 16 * t, u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
            st8(dV + off + 16 * t, u32x2{pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
        }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    bf16* __restrict__ dQ, const int32_t* __restrict__ se, const int32_t* __restrict__ q_order,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ row_ent, int L, int Hq, int Hkv,
    float scale_log2, float scale) {
    using T = Tile<D>;
    constexpr int NS = D / 32, NT = D / 16;
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * T::kBytes];
    lds_char* const smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int G = Hq / Hkv, per_kv = (int(gridDim.x) / Hq) * G;
    const int work = xcd_logical_block();
    const int hkv = work / per_kv, rank = (work % per_kv) / G, h = hkv * G + work % G;
    const int qb = q_order[rank];
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int qrow0 = qb * kBlock + 32 * wave;

    bf16x8 qf[2][NS], gf[2][NS];
    float lse2[2], dlt[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        const int qi = qrow0 + 16 * qs + n;
        lse2[qs] = LSE[int64_t(h) * L + qi] * kLog2e;
        dlt[qs] = Delta[int64_t(h) * L + qi];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[qs][s] = __builtin_bit_cast(bf16x8, ld16(Q + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g));
            gf[qs][s] = __builtin_bit_cast(bf16x8, ld16(dO + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g));
        }
    }
    f32x4 dq[2][NT];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < NT; ++t) dq[qs][t] = f32x4{0.f, 0.f, 0.f, 0.f};

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

        // two halves of 32 keys: blocks b = 2c, 2c+1 feed k-step c of dQ^T
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x4 s[2][2], dp[2][2];  // [qs][e]: lane = query column, keys 32c + 16e + 4g + 0..3
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int b = 2 * c + e;
                bf16x8 ak[NS], av[NS];
#pragma unroll
                for (int x = 0; x < NS; ++x) {
                    ak[x] = T::row_frag(kt, 16 * b + n, 4 * x + g);
                    av[x] = T::row_frag(vt, 16 * b + n, 4 * x + g);
                }
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) {
                    // dP^T accumulates onto -Delta of the lane's query
                    f32x4 cs = {0.f, 0.f, 0.f, 0.f}, cd = {-dlt[qs], -dlt[qs], -dlt[qs], -dlt[qs]};
#pragma unroll
                    for (int x = 0; x < NS; ++x) {
                        cs = mfma16x16x32(ak[x], qf[qs][x], cs);
                        cd = mfma16x16x32(av[x], gf[qs][x], cd);
                    }
                    s[qs][e] = cs;
                    dp[qs][e] = cd;
                }
            }
            bf16x8 db[2];
            auto elementwise = [&](auto masked) {
                i32x4 sek[2];
                if constexpr (decltype(masked)::value) {
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        sek[e] = *reinterpret_cast<const i32x4*>(se + kbase + 32 * c + 16 * e + 4 * g);
                }
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) {
                    const int qi = qrow0 + 16 * qs + n;
#pragma unroll
                    for (int e = 0; e < 2; ++e)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float p = fast_exp2(__builtin_fmaf(s[qs][e][r], scale_log2, -lse2[qs]));
                            if constexpr (decltype(masked)::value) {
                                const int key = kbase + 32 * c + 16 * e + 4 * g + r;
                                p = (key <= qi && qi <= sek[e][r]) ? p : 0.f;
                            }
                            dp[qs][e][r] = p * dp[qs][e][r];
                        }
                    db[qs] = to_bf16x8(dp[qs][0], dp[qs][1]);
                }
            };
            if (partial)
                elementwise(std::true_type{});
            else
                elementwise(std::false_type{});
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 a = join_tr(T::tr_frag(kt, 32 * c + 4 * g, 16 * t, n),
                                         T::tr_frag(kt, 32 * c + 16 + 4 * g, 16 * t, n));
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) dq[qs][t] = mfma16x16x32(a, db[qs], dq[qs][t]);
            }
        }

        wait_vm_all();
        __syncthreads();
    }

#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        bf16* row = dQ + int64_t(qrow0 + 16 * qs + n) * q_stride + int64_t(h) * D + 4 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 a = dq[qs][t] * scale;
            st8(row + 16 * t, u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
        }
    }
}

template <int D>
hipError_t launch_bwd_d(int phase, const bf16* Q, const bf16* K, const bf16* V, const bf16* O, const float* lse,
                        const bf16* dO, bf16* dQ, bf16* dK, bf16* dV, const int32_t* se, const MetaPtrs& mp,
                        float* delta, const AttnShape& sh, hipStream_t stream) {
    const int L = int(sh.L);
    const int64_t rows = int64_t(L) * sh.Hq;
    const float sl2 = sh.scale * kLog2e;
    float* lse2 = delta + rows;  // second half of the workspace
    if (phase == kPhaseAll || phase == kPhaseDelta)
        delta_bf16_kernel<D><<<unsigned((rows + 255) / 256), 256, 0, stream>>>(O, dO, lse, delta, lse2, L, sh.Hq);
    if (phase == kPhaseAll || phase == kPhaseDkdv)
        dkdv_bf16_kernel<D><<<unsigned(sh.nb) * unsigned(sh.Hkv), kThreads, 0, stream>>>(
            Q, K, V, dO, lse2, delta, dK, dV, se, mp.k_order, mp.col_ptr, mp.col_ent, L, sh.Hq, sh.Hkv, sl2,
            sh.scale);
    if (phase == kPhaseAll || phase == kPhaseDq)
        dq_bf16_kernel<D><<<unsigned(sh.nb) * unsigned(sh.Hq), kThreads, 0, stream>>>(
            Q, K, V, dO, lse, delta, dQ, se, mp.q_order, mp.row_ptr, mp.row_ent, L, sh.Hq, sh.Hkv, sl2, sh.scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(int phase, const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, const int32_t* se, const MetaPtrs& mp,
                           float* delta, const AttnShape& sh, hipStream_t stream) {
    const auto* Q = static_cast<const bf16*>(q);
    const auto* K = static_cast<const bf16*>(k);
    const auto* V = static_cast<const bf16*>(v);
    const auto* O = static_cast<const bf16*>(o);
    const auto* G = static_cast<const bf16*>(dout);
    auto* dQ = static_cast<bf16*>(dq);
    auto* dK = static_cast<bf16*>(dk);
    auto* dV = static_cast<bf16*>(dv);
    if (sh.D == 128) return launch_bwd_d<128>(phase, Q, K, V, O, lse, G, dQ, dK, dV, se, mp, delta, sh, stream);
    if (sh.D == 64) return launch_bwd_d<64>(phase, Q, K, V, O, lse, G, dQ, dK, dV, se, mp, delta, sh, stream);
    return hipErrorInvalidValue;
}

}  // namespace treeattn
