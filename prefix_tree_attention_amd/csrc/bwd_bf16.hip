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
// Three kernels; the whole backward runs dq, then dkdv:
//   delta: Delta for every (token, query head), for callers that run the
//          phases one by one (the whole backward computes it inside dq).
//   dkdv:  one workgroup per (key group, key/value head): a group is up
//          to four consecutive 64-key chunks sharing one subtree-end maximum
//          (the metadata's runs, cut every four chunks), so a group's keys
//          see one contiguous range of queries with little of it invisible
//          to some of them.  Wave w owns chunk w of the group and keeps its
//          V^T operands in vector registers and its dK^T, dV^T accumulators
//          in the 256 accumulation registers; K rows of the group's keys sit
//          in LDS.  It walks the group's 64-query steps for each query head
//          of the key/value head;
//          Q and dO (and -LSE / scale, -Delta) of a step go HBM -> LDS by
//          direct loads into double-buffered quad-major tiles (tile.h).
//            S = Q K^T, dP = dO V^T      (A = Q / dO rows of the tiles)
//            dV^T += dO^T P, dK^T += Q^T dS
//          (A = dO^T / Q^T by transposing LDS reads of the same tiles,
//          B = P / dS straight from the score accumulators).  Each Q / dO
//          operand read feeds two 32-key MFMAs.
//   dq:    one workgroup per (128-query block, query head) like the forward:
//            S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T,
//          K^T again by transposing reads of the K tile.  In the whole
//          backward it first forms Delta of its rows from the dO it holds
//          and one read of O, and leaves -Delta and -LSE / scale for dkdv.
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
// -Delta = -rowsum(dO * O) and -LSE / scale: the initial values of the
// dK/dV kernel's dP and S accumulators, which then leave dP - Delta and
// S - LSE / scale (so P = exp2(scale log2 e * acc))
// ---------------------------------------------------------------------------
// One 16-byte chunk per lane, D / 8 lanes per (token, head) row, so each
// row is one contiguous 2D-byte read; rows run head-major (grid y = head,
// tokens along x), so the LSE and output rows [Hq, L] are contiguous too.
template <int D>
__global__ __launch_bounds__(256) void delta_bf16_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                         const float* __restrict__ LSE, float* __restrict__ delta,
                                                         float* __restrict__ nls, float inv_scale, int L, int Hq) {
    constexpr int kLanes = D / 8;         // lanes per row
    constexpr int kRows = 256 / kLanes;   // rows per workgroup
    const int h = blockIdx.y;
    const int i = blockIdx.x * kRows + threadIdx.x / kLanes;
    const int c = threadIdx.x % kLanes;
    float acc = 0.f;
    if (i < L) {
        const int64_t off = (int64_t(i) * Hq + h) * D + 8 * c;
        const u32x4 a = ld16(O + off), b = ld16(dO + off);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc += bf16_to_float(a[w] & 0xffffu) * bf16_to_float(b[w] & 0xffffu);
            acc += bf16_to_float(a[w] >> 16) * bf16_to_float(b[w] >> 16);
        }
    }
#pragma unroll
    for (int o = kLanes / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (c == 0 && i < L) {
        const int64_t hr = int64_t(h) * L + i;
        nls[hr] = -LSE[hr] * inv_scale;
        delta[hr] = -acc;
    }
}

// direct load of 64 consecutive floats (one wave)
__device__ __forceinline__ void load_row64_async(lds_char* dst, const float* __restrict__ src, int lane) {
    dma4(src, 4u * lane, lds_addr(dst));
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
// dK^T / dV^T accumulation, D = A * B + D, with the accumulator held in
// accumulation registers (AGPRs): the 256 of them hold the 64 keys x D of
// dK and dV of one wave, which leaves the vector registers to the scores.
// The compiler's hazard recognizer does not look inside inline asm, so the
// callers keep the required distances themselves: two wait states between
// a VALU write of A or B and this read (the bf16 conversions are fenced by
// an s_nop 1), and nops before the accumulators are first read or written
// by anything else.  Consecutive updates of one accumulator by MFMAs of
// this same shape need no wait states.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(__builtin_bit_cast(i32x4, a)), "v"(__builtin_bit_cast(i32x4, b)));
}

// one workgroup per (key group, key/value head); wave w owns the group's
// 64-key chunk w
template <int D, bool kAcc, bool kRope>
__global__ __launch_bounds__(kThreads, 1) void dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLS, const float* __restrict__ Delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ dKacc, float* __restrict__ dVacc,
    const int32_t* __restrict__ se, const int32_t* __restrict__ g_order, const int32_t* __restrict__ hi64,
    const int32_t* __restrict__ hdr, int L, int Hq, int Hkv, int qb_lo, int qb_hi, float scale_log2,
    float scale, const int32_t* __restrict__ pos, const float* __restrict__ rope_tab) {
    using T = QuadTile<D>;
    constexpr int NX = D / 16;  // k-steps of S = Q K^T and dP = dO V^T
    constexpr int NT = D / 32;  // 32-row d-blocks of dK^T and dV^T
    constexpr int kStage = 2 * T::kBytes + 512;  // Q tile, dO tile, -LSE / scale [64], -Delta [64]
    constexpr int kKBytes = 4 * T::kBytes;       // K rows of the 256 keys
    __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kStage + kKBytes];
    // the two Q / dO stages first: a stage read then sits at a small
    // immediate from its per-step base
    lds_char* const smem = (lds_char*)smem_raw;
    lds_char* const ktile = smem + 2 * kStage;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 32x32x16 fragments: lane = MFMA column j32 (this lane's key within a
    // 32-key block) and k-half h
    const int j32 = lane & 31, h = lane >> 5;
    // transposing reads: 16-lane group gi takes 16 d values starting at
    // 16 (gi % 2) and query rows 4 h + 0..3 of a k-step
    const int tr_i = lane & 15;
    // work item: key/value-head major, then the key groups heaviest first
    // (the metadata bounds their number by the launch's workgroups per head)
    const int per_kv = int(gridDim.x) / Hkv;
    const int work = xcd_logical_block();
    const int hkv = work / per_kv, rank = work % per_kv;
    const int nb = L / kBlock;
    const int G = Hq / Hkv;
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    if (rank >= hdr[3]) return;  // the launch's slack beyond the groups
    // A group is nch (1..4) consecutive 64-key chunks from chunk c0; with
    // hi the largest subtree end among them (one value for all of a run's
    // chunks), its keys see the 64-query steps c0 .. hi / 64 (clipped to
    // the launch's query blocks [qb_lo, qb_hi)).
    const int gent = g_order[rank];
    const int c0 = gent & 0x3fff, nch = (gent >> 14) + 1;
    int ghi = hi64[c0];
    for (int c = 1; c < nch; ++c) ghi = max(ghi, hi64[c0 + c]);
    const int s_hi = ghi >= 0 ? min(2 * min(nb, qb_hi) - 1, ghi / kChunk) : -1;
    const int s_lo = max(c0, 2 * qb_lo);
    const int nsteps = (s_hi >= s_lo ? s_hi - s_lo + 1 : 0) * G;
    if (kAcc && nsteps == 0) return;  // nothing to add
    // wave w owns chunk c0 + w; a wave past the group's chunks shadows its
    // first chunk (in-range reads) and stores nothing
    const bool active = wave < nch;
    const int cw = c0 + (active ? wave : 0);

    // V^T operands (B of dP) in registers: lane holds key
    // 64 cw + 32 kk + j32, d = 16 x + 8 h .. +7 for k-step x.
    // K^T operands (B of S) are read from the K rows in LDS with the same
    // offsets as the Q rows.
    bf16x8 vf[2][NX];
    int key[2], sek[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        key[kk] = kChunk * cw + 32 * kk + j32;
        sek[kk] = se[key[kk]];
        const int64_t base = int64_t(key[kk]) * kv_stride + hkv * D + 8 * h;
#pragma unroll
        for (int x = 0; x < NX; ++x) vf[kk][x] = __builtin_bit_cast(bf16x8, ld16(V + base + 16 * x));
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = kChunk * (c0 + (q4 < nch ? q4 : 0));
        T::load_async(ktile + q4 * T::kBytes, K + int64_t(r0) * kv_stride + hkv * D, int(kv_stride), wave, lane);
    }
    // Operand read offsets, one base per lane and pattern: the row-major
    // read of k-step x (chunk 2 x + h of row j32) is at rlane + px(x); the
    // transposing read of d-block t (rows 4 h + 8 v + 0..3 of a 16-row
    // k-step, chunk pair 2 t + (lane / 16) % 2) at tlane + R8 v + QS t.
    // Every other term is an immediate.
    int rlane = T::rb(j32) + 16 * h;
    int tlane = T::rb(4 * h) + 32 * ((lane >> 4) & 1) + T::tr_lane(tr_i);
    auto roff = [&](int x) { return rlane + T::px(x); };
    auto toff = [&](int t, int v) { return tlane + T::kR8 * v + T::kQs * t; };
    // dK^T, dV^T accumulators of key block kk: d-block t, register r =
    // d 32 t + 8 (r / 4) + 4 h + r % 4
    f32x16 dk[2][NT], dv[2][NT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) dk[kk][t][r] = dv[kk][t][r] = 0.f;
    // nops that every accumulator depends on (see mfma32_agpr)
#define TREEATTN_FENCE_ACC(NOPS)                                                                             \
    do {                                                                                                     \
        if constexpr (NT == 4)                                                                               \
            asm volatile(NOPS                                                                                \
                         : "+a"(dk[0][0]), "+a"(dk[0][1]), "+a"(dk[0][2]), "+a"(dk[0][3]), "+a"(dk[1][0]),  \
                           "+a"(dk[1][1]), "+a"(dk[1][2]), "+a"(dk[1][3]), "+a"(dv[0][0]), "+a"(dv[0][1]),   \
                           "+a"(dv[0][2]), "+a"(dv[0][3]), "+a"(dv[1][0]), "+a"(dv[1][1]), "+a"(dv[1][2]),   \
                           "+a"(dv[1][3]));                                                                  \
        else                                                                                                 \
            asm volatile(NOPS                                                                                \
                         : "+a"(dk[0][0]), "+a"(dk[0][1]), "+a"(dk[1][0]), "+a"(dk[1][1]), "+a"(dv[0][0]),  \
                           "+a"(dv[0][1]), "+a"(dv[1][0]), "+a"(dv[1][1]));                                  \
    } while (0)
    static_assert(NT == 4 || NT == 2, "D is 128 or 64");
    TREEATTN_FENCE_ACC("s_nop 1");  // zeroing writes -> first MFMA read

    const int kmax_w = kChunk * cw + 63;
    int lo_w = min(sek[0], sek[1]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lo_w = min(lo_w, __shfl_xor(lo_w, o));
    lo_w = __builtin_amdgcn_readfirstlane(lo_w);
    const int qs32 = int(q_stride);
    auto qtile = [&](int buf) { return smem + buf * kStage; };
    auto gtile = [&](int buf) { return smem + buf * kStage + T::kBytes; };
    auto lsev = [&](int buf) { return smem + buf * kStage + 2 * T::kBytes; };
    auto dlv = [&](int buf) { return smem + buf * kStage + 2 * T::kBytes + 256; };
    // Steps run over the query heads of the group fastest, then the 64-query
    // steps from the last down, so the groups in flight on an XCD read the
    // same Q / dO tiles at about the same time.
    struct StepPos {
        int qbase, head;
    };
    auto advance = [&](StepPos& p) {
        if (++p.head == G) {
            p.head = 0;
            p.qbase -= kStep;
        }
    };
    const uint32_t q_row_bytes = uint32_t(q_stride) * 2u;
    auto issue = [&](const StepPos& p, int buf) {
        const int hq = hkv * G + p.head;
        const uint64_t off = uint64_t(uint32_t(p.qbase)) * q_row_bytes + uint32_t(hq * D * 2);
        T::load_async(qtile(buf), reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(Q) + off), qs32, wave,
                      lane);
        T::load_async(gtile(buf), reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(dO) + off), qs32,
                      wave, lane);
        if (wave == 0) load_row64_async(lsev(buf), NLS + int64_t(hq) * L + p.qbase, lane);
        if (wave == 1) load_row64_async(dlv(buf), Delta + int64_t(hq) * L + p.qbase, lane);
    };
    StepPos cur{s_hi * kChunk, 0}, nxt{s_hi * kChunk, 0};
    // the first two steps' tiles; step st issues step st + 2's
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (i < nsteps) {
            issue(nxt, i);
            advance(nxt);
        }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        consume(sek[kk]);
#pragma unroll
        for (int x = 0; x < NX; ++x) consume(vf[kk][x]);
    }
    wait_vm_all();
    __syncthreads();

    const lds_char* kt = ktile + wave * T::kBytes;
    struct SOps {
        bf16x8 aq, k0, k1;
    };
    // k-step x of S: Q rows of half c of buffer buf and the wave's two
    // 32-key K blocks
    auto rd_s = [&](int buf, int c, int x) {
        const int ro = roff(x);
        return SOps{T::frag_at(qtile(buf) + 2 * c * T::kGs, ro), T::frag_at(kt, ro),
                    T::frag_at(kt + 2 * T::kGs, ro)};
    };
    // S starts at -LSE / scale and dP at -Delta, so they leave
    // S - LSE / scale and dP - Delta; register r of a score accumulator
    // holds query 32 c + 8 (r / 4) + 4 h + r % 4 against key 32 kk + j32
    auto rd_init = [&](int buf, int c, f32x16& nl, f32x16& nd) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                lsev(buf) + 4 * (32 * c + 8 * j + 4 * h));
            const f32x4 b = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                dlv(buf) + 4 * (32 * c + 8 * j + 4 * h));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                nl[4 * j + i] = a[i];
                nd[4 * j + i] = b[i];
            }
        }
    };
    // the first reads of a step (made at the end of the previous one)
    f32x16 nl, nd;
    SOps so[NX];
    rd_init(0, 0, nl, nd);
    so[0] = rd_s(0, 0, 0);
    so[1] = rd_s(0, 0, 1);

    // One step is 64 queries in two halves of 32.  Per half the MFMA stream
    // is S (NX), dP (NX), then dV (2 NT), dK (2 NT) and both again (4 NT);
    // the exponentials run between the dP MFMAs and dS between the first
    // gradient MFMAs, so the matrix core keeps work queued while the vector
    // unit runs (one wave per SIMD hides nothing by itself).  Scheduling
    // barriers pin that order; each group issues the LDS reads of the group
    // two ahead.  The step's barrier sits two gradient groups before its
    // end, once its last reads have returned, so the next step's tiles are
    // requested and its first operands read while those groups run.
#define TREEATTN_SCHED() __builtin_amdgcn_sched_barrier(0)
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int qbase = cur.qbase;
        advance(cur);
        const lds_char* qt = qtile(buf);
        const lds_char* gt = gtile(buf);

        // k-step x of dP: dO rows of the half
        auto rd_g = [&](int c, int x) { return T::frag_at(gt + 2 * c * T::kGs, roff(x)); };
        // d-block t, k-step m of the gradients from the dO tile (dO^T) or
        // the Q tile (Q^T): rows 32 c + 16 m + 4 h + {0..3, 8..11}
        auto rd_tr = [&](const lds_char* tile, int c, int t, int m) {
            const int rb = (2 * c + m) * T::kGs;
            return join_tr(T::tr_at(tile + rb, toff(t, 0)), T::tr_at(tile + rb, toff(t, 1)));
        };
        auto cvt8 = [](const f32x16& s, int m) {
            return to_bf16x8(f32x4{s[8 * m], s[8 * m + 1], s[8 * m + 2], s[8 * m + 3]},
                             f32x4{s[8 * m + 4], s[8 * m + 5], s[8 * m + 6], s[8 * m + 7]});
        };

        constexpr int kExp = 32 / NX;     // exponentials per dP k-step
        constexpr int kDs = 16 / NT / 2;  // dS products per gradient MFMA pair
        // opaque per step, so the offsets are formed at each use rather than
        // hoisted out of the loop into one register each
        asm volatile("" : "+v"(rlane), "+v"(tlane));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x16 sc[2], dp[2];
            bf16x8 ag[NX], pb[2][2], db[2][2];
            bf16x8 tg[2][NT], tq[2][NT];  // dO^T, Q^T of k-step m, d-block t
            // gradient operand reads in the order they are consumed: dO^T of
            // k-step 0 (dV), Q^T of k-step 0 (dK), then both of k-step 1
            auto rd_unit = [&](int u) {
                if (u < NT) {
                    tg[0][u] = rd_tr(gt, c, u, 0);
                } else if (u < 2 * NT) {
                    tq[0][u - NT] = rd_tr(qt, c, u - NT, 0);
                } else {
                    tg[1][u - 2 * NT] = rd_tr(gt, c, u - 2 * NT, 1);
                    tq[1][u - 2 * NT] = rd_tr(qt, c, u - 2 * NT, 1);
                }
            };
            TREEATTN_SCHED();
            // S = Q K^T
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                if (x + 2 < NX)
                    so[x + 2] = rd_s(buf, c, x + 2);
                else
                    ag[x + 2 - NX] = rd_g(c, x + 2 - NX);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    sc[kk] = mfma32x32x16(so[x].aq, kk ? so[x].k1 : so[x].k0, x == 0 ? nl : sc[kk]);
                TREEATTN_SCHED();
            }
            // dP = dO V^T, with P = exp2(scale log2e (S - LSE / scale)) of
            // 32 / NX scores after each k-step; the subtree-interval
            // predicate only where the half is partial for this wave:
            // register r is query q0 + o_r, o_r = 8 (r / 4) + r % 4, and
            // key <= q <= se[key]  <=>  key - q0 <= o_r <= se[key] - q0
            auto dp_exp = [&](auto masked_t) {
                constexpr bool kMasked = decltype(masked_t)::value;
                // Opaque and different in the two variants, so the common
                // work (reads, scaling, conversions) stays inside each rather
                // than being hoisted above the branch or sunk below it, out
                // of reach of the dP MFMAs.
                float sl = scale_log2;
                if constexpr (kMasked)
                    asm volatile("; partial half" : "+v"(rlane), "+v"(tlane), "+s"(sl));
                else
                    asm volatile("; full half" : "+v"(rlane), "+v"(tlane), "+s"(sl));
                TREEATTN_SCHED();
                // the lane's visible offsets o form one interval per key,
                // [key - q0, se[key] - q0]; bit o of vis[kk] is set for
                // those in 0..31, so a score is kept by one sign-extended
                // bit extract and an AND (a cleared p is +0)
                uint32_t vis[2] = {0u, 0u};
                if constexpr (kMasked) {
                    const int q0 = qbase + 32 * c + 4 * h;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int lo = max(key[kk] - q0, 0), hi = min(sek[kk] - q0, 31);
                        const int width = hi - lo + 1;
                        vis[kk] = width >= 32 ? ~0u : width <= 0 ? 0u : ((1u << width) - 1u) << lo;
                    }
                }
                auto ex = [&](int e) {
                    const int kk = e >> 4, r = e & 15;
                    float p = fast_exp2(sc[kk][r] * sl);
                    if constexpr (kMasked) {
                        const int o = 8 * (r / 4) + r % 4;
                        int32_t keep = __builtin_amdgcn_sbfe(int32_t(vis[kk]), o, 1);
                        // opaque, so the AND stays an AND instead of a
                        // compare and select (and stays compiler-visible:
                        // it reads a transcendental result, which needs a
                        // wait state the compiler inserts only for its own
                        // instructions)
                        asm("" : "+v"(keep));
                        p = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p) & uint32_t(keep));
                    }
                    sc[kk][r] = p;
                    if ((e & 7) == 7) pb[kk][(e >> 3) & 1] = cvt8(sc[kk], (e >> 3) & 1);
                };
#pragma unroll
                for (int x = 0; x < NX; ++x) {
                    if (x + 2 < NX)
                        ag[x + 2] = rd_g(c, x + 2);
                    else
                        rd_unit(x + 2 - NX);
                    dp[0] = mfma32x32x16(ag[x], vf[0][x], x == 0 ? nd : dp[0]);
#pragma unroll
                    for (int e = 0; e < kExp / 2; ++e) ex(kExp * x + e);
                    dp[1] = mfma32x32x16(ag[x], vf[1][x], x == 0 ? nd : dp[1]);
#pragma unroll
                    for (int e = kExp / 2; e < kExp; ++e) ex(kExp * x + e);
                    TREEATTN_SCHED();
                }
                // also the two wait states between the P conversions (VALU
                // writes) and the asm MFMAs that read them
                if constexpr (kMasked)
                    asm volatile("s_nop 1 ; partial half end"
                                 : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]));
                else
                    asm volatile("s_nop 1 ; full half end"
                                 : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]));
            };
            // A half is full (no mask) for this wave when every one of its 64
            // keys precedes every query of the half and every query ends
            // inside every key's subtree: a test on the wave's last key and
            // smallest subtree end (pads count -1, so a wave holding one
            // always masks).
            const int q0c = qbase + 32 * c;
            if (q0c >= kmax_w && q0c + 31 <= lo_w)
                dp_exp(std::false_type{});
            else
                dp_exp(std::true_type{});
            TREEATTN_SCHED();
            // dS = P (dP - Delta), 16 products per k-step m (queries
            // 32 c + 16 m + ..), spread over the gradient MFMAs before the
            // ones that read them; the conversions are VALU writes that the
            // asm MFMAs read, hence the s_nop 1 fences
            auto ds_part = [&](int m, int t, int kk) {
#pragma unroll
                for (int i = 0; i < kDs; ++i) {
                    const int e = (2 * t + kk) * kDs + i;  // 0..15
                    const int k2 = e >> 3, r = 8 * m + (e & 7);
                    dp[k2][r] *= sc[k2][r];
                    if ((e & 7) == 7) db[k2][m] = cvt8(dp[k2], m);
                }
            };
            // dV^T += dO^T P, k-step 0, with dS of k-step 0
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                rd_unit(t + 2);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    mfma32_agpr(dv[kk][t], tg[0][t], pb[kk][0]);
                    ds_part(0, t, kk);
                }
                TREEATTN_SCHED();
            }
            asm("s_nop 1" : "+v"(db[0][0]), "+v"(db[1][0]));
            TREEATTN_SCHED();
            // dK^T += Q^T dS, k-step 0, with dS of k-step 1
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                rd_unit(NT + t + 2);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    mfma32_agpr(dk[kk][t], tq[0][t], db[kk][0]);
                    ds_part(1, t, kk);
                }
                TREEATTN_SCHED();
            }
            asm("s_nop 1" : "+v"(db[0][1]), "+v"(db[1][1]));
            TREEATTN_SCHED();
            // k-step 1 of both, then the next half's first reads; in the
            // second half, the step's barrier once the last reads of this
            // buffer have returned, then the tiles of step st + 2 into it
            // and the first reads of step st + 1 (stale but in-bounds LDS
            // after the last step, never used)
            constexpr int kBarT = NT - 2;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int u = 2 * NT + t + 2;
                if (c == 1 && t == kBarT) {
                    wait_vm_all();
                    __syncthreads();
                    if (st + 2 < nsteps) {
                        issue(nxt, buf);
                        advance(nxt);
                    }
                }
                if (u < 3 * NT) {
                    rd_unit(u);
                } else if (u == 3 * NT) {
                    rd_init(c == 0 ? buf : buf ^ 1, c ^ 1, nl, nd);
                } else {
                    so[0] = rd_s(c == 0 ? buf : buf ^ 1, c ^ 1, 0);
                    so[1] = rd_s(c == 0 ? buf : buf ^ 1, c ^ 1, 1);
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    mfma32_agpr(dv[kk][t], tg[1][t], pb[kk][1]);
                    mfma32_agpr(dk[kk][t], tq[1][t], db[kk][1]);
                }
                TREEATTN_SCHED();
            }
        }
    }
#undef TREEATTN_SCHED
    TREEATTN_FENCE_ACC("s_nop 7\n\ts_nop 7\n\ts_nop 7");  // last MFMA writes -> the reads below
#undef TREEATTN_FENCE_ACC

    // lane holds key 32 kk + j32 of the wave, d = 32 t + 8 j + 4 h + 0..3 in
    // registers 4 j + 0..3
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        if (!active) continue;
        const int64_t off = int64_t(key[kk]) * kv_stride + hkv * D + 4 * h;
        if constexpr (kRope) {
            // the gradient w.r.t. the unrotated key: rotate back by the key's
            // tree position; d = 32 t + 8 j + 4 h + r pairs with t + NT/2
            const float* cs = rope_tab + (int64_t(pos[key[kk]]) * (D / 2) + 4 * h) * 2;
#pragma unroll
            for (int t = 0; t < NT / 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4* t4 = reinterpret_cast<const f32x4*>(cs + 2 * (32 * t + 8 * j));
                    const f32x4 c0 = t4[0], c1 = t4[1];
                    const float c[4] = {c0[0], c0[2], c1[0], c1[2]}, sn[4] = {c0[1], c0[3], c1[1], c1[3]};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x1 = dk[kk][t][4 * j + r], x2 = dk[kk][t + NT / 2][4 * j + r];
                        rope_pair<true>(x1, x2, c[r], sn[r]);
                        dk[kk][t][4 * j + r] = x1;
                        dk[kk][t + NT / 2][4 * j + r] = x2;
                    }
                }
        }
        if constexpr (kAcc) {
            // add to float32 accumulators (this workgroup owns these keys'
            // rows for the launch, so a plain read-modify-write)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 32 * t + 8 * j;
                    f32x4* ak = reinterpret_cast<f32x4*>(dKacc + off + d0);
                    f32x4* av = reinterpret_cast<f32x4*>(dVacc + off + d0);
                    const f32x4 xk = *ak, xv = *av;
                    *ak = f32x4{xk[0] + dk[kk][t][4 * j] * scale, xk[1] + dk[kk][t][4 * j + 1] * scale,
                                xk[2] + dk[kk][t][4 * j + 2] * scale, xk[3] + dk[kk][t][4 * j + 3] * scale};
                    *av = f32x4{xv[0] + dv[kk][t][4 * j], xv[1] + dv[kk][t][4 * j + 1], xv[2] + dv[kk][t][4 * j + 2],
                                xv[3] + dv[kk][t][4 * j + 3]};
                }
            continue;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * t + 8 * j;
                st8(dK + off + d0, u32x2{pack_bf16x2(dk[kk][t][4 * j] * scale, dk[kk][t][4 * j + 1] * scale),
                                         pack_bf16x2(dk[kk][t][4 * j + 2] * scale, dk[kk][t][4 * j + 3] * scale)});
                st8(dV + off + d0, u32x2{pack_bf16x2(dv[kk][t][4 * j], dv[kk][t][4 * j + 1]),
                                         pack_bf16x2(dv[kk][t][4 * j + 2], dv[kk][t][4 * j + 3])});
            }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, bool kDelta, bool kRope>
__global__ __launch_bounds__(kThreads, 2) void dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ Delta, float* __restrict__ NLS, bf16* __restrict__ dQ, const int32_t* __restrict__ se,
    const int32_t* __restrict__ q_order, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ row_ent,
    int L, int Hq, int Hkv, float scale_log2, float scale, const int32_t* __restrict__ pos,
    const float* __restrict__ rope_tab) {
    using T = QuadTile<D>;
    constexpr int NS = D / 32, NT = D / 16;
    // K and V tiles and the keys' subtree ends, double-buffered
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * T::kBytes + 2 * 4 * kStep];
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
    u32x4 of[2][NS];  // O chunks matching gf, for Delta (kDelta)
    float lse_raw[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        const int qi = qrow0 + 16 * qs + n;
        const int64_t hr = int64_t(h) * L + qi;
        const float lse = LSE[hr];
        lse2[qs] = lse * kLog2e;
        if constexpr (!kDelta) dlt[qs] = -Delta[hr];  // stored negated
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[qs][s] = __builtin_bit_cast(bf16x8, ld16(Q + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g));
            gf[qs][s] = __builtin_bit_cast(bf16x8, ld16(dO + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g));
        }
        if constexpr (kDelta) {
            lse_raw[qs] = lse;
#pragma unroll
            for (int s = 0; s < NS; ++s) of[qs][s] = ld16(O + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g);
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
    auto serow = [&](int buf) { return smem + 4 * T::kBytes + buf * 4 * kStep; };
    const char* const Kh = reinterpret_cast<const char*>(K + int64_t(hkv) * D);
    const char* const Vh = reinterpret_cast<const char*>(V + int64_t(hkv) * D);
    const uint32_t kv_row_bytes = uint32_t(kv_stride) * 2u;
    auto issue = [&](int st, int buf) {
        const int kbase = (row_ent[beg + (st >> 1)] >> 1) * kBlock + kStep * (st & 1);
        const uint64_t off = uint64_t(uint32_t(kbase)) * kv_row_bytes;
        T::load_async(ktile(buf), reinterpret_cast<const bf16*>(Kh + off), kvs, wave, lane);
        T::load_async(vtile(buf), reinterpret_cast<const bf16*>(Vh + off), kvs, wave, lane);
        // the keys' subtree ends ride with the tiles (wave w stages 16 of
        // them), so the partial-tile mask reads LDS instead of issuing
        // global loads whose wait would also drain the prefetch
        if (lane < 16) dma4(se + kbase + 16 * wave, 4u * lane, lds_addr(serow(buf) + 64 * wave));
    };
    if (nsteps > 0) issue(0, 0);
    if constexpr (kDelta) {
        // Delta_i = dO_i . O_i from the dO chunks this lane already holds
        // and the matching O chunks, formed while the first tiles load: the
        // four lanes n + 16 g of a query hold its D elements, so two
        // exchanges finish the sum.  Lane g = 0 leaves -Delta and
        // -LSE / scale for the dK/dV kernel.
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 a = of[qs][s], b = __builtin_bit_cast(u32x4, gf[qs][s]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc += bf16_to_float(a[w] & 0xffffu) * bf16_to_float(b[w] & 0xffffu);
                    acc += bf16_to_float(a[w] >> 16) * bf16_to_float(b[w] >> 16);
                }
            }
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            dlt[qs] = acc;
            if (g == 0) {
                const int64_t hr = int64_t(h) * L + qrow0 + 16 * qs + n;
                Delta[hr] = -acc;
                NLS[hr] = -lse_raw[qs] / scale;
            }
        }
    }
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        consume(lse2[qs]);
        consume(dlt[qs]);
#pragma unroll
        for (int x = 0; x < NS; ++x) {
            consume(qf[qs][x]);
            consume(gf[qs][x]);
        }
    }
    wait_vm_all();
    __syncthreads();

    // LDS offsets of this lane's operand reads (quad-major tiles): K and V
    // rows 16 b + n, chunk 4 x + g, at rlane + 16-row moves + QS x; K^T
    // rows 4 g + 0..3 of each 16-row k-half, elements 16 t + 4 (n % 4) ..,
    // at tlane + 16-row moves + px(t)
    const int rlane = T::rb(n) + 16 * g;
    const int tlane = T::rb(4 * g) + T::tr_lane(n);
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
                    ak[x] = T::frag_at(kt + b * T::kGs, rlane + T::kQs * x);
                    av[x] = T::frag_at(vt + b * T::kGs, rlane + T::kQs * x);
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
                        sek[e] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
                            serow(buf) + 4 * (32 * c + 16 * e + 4 * g));
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
                const bf16x8 a = join_tr(T::tr_at(kt + 2 * c * T::kGs, tlane + T::px(t)),
                                         T::tr_at(kt + (2 * c + 1) * T::kGs, tlane + T::px(t)));
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) dq[qs][t] = mfma16x16x32(a, db[qs], dq[qs][t]);
            }
        }

        wait_vm_all();
        __syncthreads();
    }

#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        const int qi = qrow0 + 16 * qs + n;
        if constexpr (kRope) {
            // the gradient w.r.t. the unrotated query: rotate back by the
            // query's tree position; d = 16 t + 4 g + r pairs with t + NT/2
            const float* cs = rope_tab + (int64_t(pos[qi]) * (D / 2) + 4 * g) * 2;
#pragma unroll
            for (int t = 0; t < NT / 2; ++t) {
                const f32x4* t4 = reinterpret_cast<const f32x4*>(cs + 32 * t);
                const f32x4 c0 = t4[0], c1 = t4[1];
                const float c[4] = {c0[0], c0[2], c1[0], c1[2]}, sn[4] = {c0[1], c0[3], c1[1], c1[3]};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x1 = dq[qs][t][r], x2 = dq[qs][t + NT / 2][r];
                    rope_pair<true>(x1, x2, c[r], sn[r]);
                    dq[qs][t][r] = x1;
                    dq[qs][t + NT / 2][r] = x2;
                }
            }
        }
        bf16* row = dQ + int64_t(qi) * q_stride + int64_t(h) * D + 4 * g;
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
                        float* delta, const AttnShape& sh, hipStream_t stream, const RowSel& sel,
                        const RopeArgs& rope) {
    const int L = int(sh.L);
    const int64_t rows = int64_t(L) * sh.Hq;
    const float sl2 = sh.scale * kLog2e;
    float* nls = delta + rows;  // second half of the workspace
    // dQ work items: (query block of the list, query head); dK/dV: (key
    // group of the heaviest-first order, key/value head), with the slack of
    // dkdv_workgroups over the groups' number
    const int32_t* q_order = sel.q_list ? sel.q_list : mp.q_order;
    const unsigned dq_grid = (sel.q_list ? unsigned(sel.n_q) : unsigned(sh.nb)) * unsigned(sh.Hq);
    const unsigned n_wg = sel.n_wg >= 0 ? unsigned(sel.n_wg) : unsigned(dkdv_workgroups(int64_t(sh.nb) * 2));
    const int qb_lo = sel.qb_lo, qb_hi = sel.qb_hi;
    if (phase == kPhaseDelta)
        delta_bf16_kernel<D><<<dim3(unsigned((L + 256 / (D / 8) - 1) / (256 / (D / 8))), unsigned(sh.Hq)), 256, 0,
                               stream>>>(O, dO, lse, delta, nls, 1.0f / sh.scale, L, sh.Hq);
    // the whole backward: dQ first, computing Delta itself and leaving it
    // (with -LSE / scale) for dK/dV, which saves a pass over O and dO
    const bool fuse_rope = rope.tab != nullptr;
    if (fuse_rope && (sel.dk_acc || phase == kPhaseDq)) return hipErrorInvalidValue;  // not combined
    if ((phase == kPhaseAll || phase == kPhaseDqDelta) && dq_grid > 0) {
        if (fuse_rope)
            dq_bf16_kernel<D, true, true><<<dq_grid, kThreads, 0, stream>>>(
                Q, K, V, dO, O, lse, delta, nls, dQ, se, q_order, mp.row_ptr, mp.row_ent, L, sh.Hq, sh.Hkv, sl2,
                sh.scale, rope.pos, rope.tab);
        else
            dq_bf16_kernel<D, true, false><<<dq_grid, kThreads, 0, stream>>>(
                Q, K, V, dO, O, lse, delta, nls, dQ, se, q_order, mp.row_ptr, mp.row_ent, L, sh.Hq, sh.Hkv, sl2,
                sh.scale, nullptr, nullptr);
    }
    if ((phase == kPhaseAll || phase == kPhaseDkdv) && n_wg > 0) {
        const dim3 grid(n_wg * unsigned(sh.Hkv));
        if (sel.dk_acc)
            dkdv_bf16_kernel<D, true, false><<<grid, kThreads, 0, stream>>>(
                Q, K, V, dO, nls, delta, dK, dV, sel.dk_acc, sel.dv_acc, se, mp.g_order, mp.hi64, mp.hdr, L,
                sh.Hq, sh.Hkv, qb_lo, qb_hi, sl2, sh.scale, nullptr, nullptr);
        else if (fuse_rope)
            dkdv_bf16_kernel<D, false, true><<<grid, kThreads, 0, stream>>>(
                Q, K, V, dO, nls, delta, dK, dV, nullptr, nullptr, se, mp.g_order, mp.hi64, mp.hdr, L,
                sh.Hq, sh.Hkv, qb_lo, qb_hi, sl2, sh.scale, rope.pos, rope.tab);
        else
            dkdv_bf16_kernel<D, false, false><<<grid, kThreads, 0, stream>>>(
                Q, K, V, dO, nls, delta, dK, dV, nullptr, nullptr, se, mp.g_order, mp.hi64, mp.hdr, L,
                sh.Hq, sh.Hkv, qb_lo, qb_hi, sl2, sh.scale, nullptr, nullptr);
    }
    if (phase == kPhaseDq && dq_grid > 0)
        dq_bf16_kernel<D, false, false><<<dq_grid, kThreads, 0, stream>>>(
            Q, K, V, dO, O, lse, delta, nls, dQ, se, q_order, mp.row_ptr, mp.row_ent, L, sh.Hq, sh.Hkv, sl2,
            sh.scale, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(int phase, const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, const int32_t* se, const MetaPtrs& mp,
                           float* delta, const AttnShape& sh, hipStream_t stream, const RowSel& sel,
                           const RopeArgs& rope) {
    const auto* Q = static_cast<const bf16*>(q);
    const auto* K = static_cast<const bf16*>(k);
    const auto* V = static_cast<const bf16*>(v);
    const auto* O = static_cast<const bf16*>(o);
    const auto* G = static_cast<const bf16*>(dout);
    auto* dQ = static_cast<bf16*>(dq);
    auto* dK = static_cast<bf16*>(dk);
    auto* dV = static_cast<bf16*>(dv);
    if (sh.D == 128) return launch_bwd_d<128>(phase, Q, K, V, O, lse, G, dQ, dK, dV, se, mp, delta, sh, stream, sel, rope);
    if (sh.D == 64) return launch_bwd_d<64>(phase, Q, K, V, O, lse, G, dQ, dK, dV, se, mp, delta, sh, stream, sel, rope);
    return hipErrorInvalidValue;
}

}  // namespace treeattn
