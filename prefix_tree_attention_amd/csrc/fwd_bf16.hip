// Forward tree attention, bf16 in / fp32 accumulate, gfx950 MFMA.
//
// What it computes (AReaL tree-training guide, packing figure: a token
// attends to itself and its ancestors only; key j is visible to query i iff
// j <= i <= se[j] in the pre-order layout):
//   O_i = sum_{j in A(i)} softmax_j(scale q_i.k_j) v_j,
//   LSE_i = ln sum_{j in A(i)} exp(scale q_i.k_j).
//
// Work decomposition: one workgroup (4 waves) per (128-query block, query
// head); wave w owns queries 32w..32w+31 of the block, one query per MFMA
// column (32x32x16 MFMAs).  The workgroup walks only the nonempty key tiles
// of its query block (row list of the metadata), 64 keys per pipeline step.
// K and V of a step go HBM -> LDS by direct loads into swizzled two-deep
// rings (tile.h) while earlier steps compute.  Partial tiles apply the
// subtree-interval predicate; full tiles skip it.
//
// Products are computed transposed: S^T = K Q^T (A = K rows from LDS, B =
// Q^T held in registers), O^T = V^T P^T (A = V^T read from the row-major V
// tile by transposing LDS loads, B = P^T taken straight from the S^T
// accumulators).  Each lane thus owns one query column, keys split over
// the lane pair l, l ^ 32, so softmax statistics need an in-lane reduction
// plus one cross-lane step, and the rescaling of O^T is per lane.  k-step m
// of the PV product covers keys 16m .. 16m + 15 of the step, and the
// transposing reads of V take exactly the key rows those accumulator
// registers hold.  Softmax runs in base 2 with scale*log2(e) folded into
// one FMA.

#include <cmath>
#include <type_traits>

#include "device.h"
#include "mfma.h"
#include "tile.h"

namespace treeattn {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = kTileRows;  // keys per pipeline step
constexpr float kRescaleSlack = 8.f;  // log2 units: p <= 256 between rescales

template <int D, bool kRope>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ se,
    const int32_t* __restrict__ q_order, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ row_ent, int L, int Hq, int Hkv, float scale_log2,
    const int32_t* __restrict__ pos, const float* __restrict__ rope_tab, bf16* __restrict__ Qrot) {
    using T = Tile<D>;
    constexpr int NX = D / 16;  // k-steps of S^T = K Q^T
    constexpr int NT = D / 32;  // 32-row d-blocks of O^T
    // K and V tiles and the keys' subtree ends, double-buffered
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * T::kBytes + 2 * 4 * kStep];
    lds_char* const smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 32x32x16 fragments: lane = MFMA column j32 (this lane's query) and k-half h
    const int j32 = lane & 31, h = lane >> 5;
    const int tr_e = 16 * ((lane >> 4) & 1), tr_i = lane & 15;
    // work item: key/value-head major, then query blocks in the metadata's
    // order (descending position), then the query heads of the group
    const int G = Hq / Hkv, per_kv = (int(gridDim.x) / Hq) * G;
    const int work = xcd_logical_block();
    const int hkv = work / per_kv, rank = (work % per_kv) / G, h_q = hkv * G + work % G;
    const int qb = q_order[rank];
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int qi = qb * kBlock + 32 * wave + j32;  // this lane's query

    // Q^T operand (B of S^T): lane holds query qi, d = 16 x + 8 h .. +7
    bf16x8 qf[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x)
        qf[x] = __builtin_bit_cast(bf16x8, ld16(Q + int64_t(qi) * q_stride + int64_t(h_q) * D + 16 * x + 8 * h));
    if constexpr (kRope) {
        // rotary embedding by the query's tree position, on the operand as it
        // is loaded: chunk x holds d = 16 x + 8 h + u, its rotation partners
        // d + D/2 are chunk x + NX/2 of the same lane; the rotated query also
        // goes to Qrot for the backward
        const float* cs = rope_tab + (int64_t(pos[qi]) * (D / 2) + 8 * h) * 2;
#pragma unroll
        for (int x = 0; x < NX / 2; ++x) {
            const f32x4* t4 = reinterpret_cast<const f32x4*>(cs + 32 * x);
            const f32x4 c0 = t4[0], c1 = t4[1], c2 = t4[2], c3 = t4[3];
            const float c[8] = {c0[0], c0[2], c1[0], c1[2], c2[0], c2[2], c3[0], c3[2]};
            const float sn[8] = {c0[1], c0[3], c1[1], c1[3], c2[1], c2[3], c3[1], c3[3]};
            f32x4 a0, a1, b0, b1;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float x1 = float(qf[x][u]), x2 = float(qf[x + NX / 2][u]);
                rope_pair<false>(x1, x2, c[u], sn[u]);
                a0[u] = x1;
                b0[u] = x2;
                float y1 = float(qf[x][u + 4]), y2 = float(qf[x + NX / 2][u + 4]);
                rope_pair<false>(y1, y2, c[u + 4], sn[u + 4]);
                a1[u] = y1;
                b1[u] = y2;
            }
            qf[x] = to_bf16x8(a0, a1);
            qf[x + NX / 2] = to_bf16x8(b0, b1);
        }
        bf16* qr = Qrot + int64_t(qi) * q_stride + int64_t(h_q) * D + 8 * h;
#pragma unroll
        for (int x = 0; x < NX; ++x) st16(qr + 16 * x, __builtin_bit_cast(u32x4, qf[x]));
    }
    // loop-invariant swizzled LDS offsets of this lane's operand reads
    int roff[NX];  // K rows: row j32, chunk 2 x + h
#pragma unroll
    for (int x = 0; x < NX; ++x) roff[x] = T::slot(j32, 2 * x + h);
    int toff[NT][2];  // V^T: d-block t, key rows 4 h + 8 v + 0..3
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 2; ++v) toff[t][v] = T::tr_offset(4 * h + 8 * v, 32 * t + tr_e, tr_i);

    // O^T accumulators: block t, register r = d 32 t + 8 (r / 4) + 4 h + r % 4
    f32x16 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
    // running max (scaled units) and this lane's partial row sum
    float m_run = -INFINITY, l_run = 0.f;

    const int beg = row_ptr[qb], nsteps = 2 * (row_ptr[qb + 1] - beg);
    const int kvs = int(kv_stride);
    // Software pipeline: while step st runs its softmax and P V, the S^T of
    // step st + 1 is computed, so the MFMA unit has independent work while
    // the wave does its exp / row-sum VALU work.  K and V therefore sit in
    // separate two-deep rings: at step st, V(st) and K(st + 1) (with its
    // keys' subtree ends) are resident while K(st + 2) and V(st + 1) load.
    auto ktile = [&](int st) { return smem + (st & 1) * T::kBytes; };
    auto vtile = [&](int st) { return smem + (2 + (st & 1)) * T::kBytes; };
    auto serow = [&](int st) { return smem + 4 * T::kBytes + (st & 1) * 4 * kStep; };
    // byte addresses: a step's tiles start at (head base) + kbase * row bytes
    const char* const Kh = reinterpret_cast<const char*>(K + int64_t(hkv) * D);
    const char* const Vh = reinterpret_cast<const char*>(V + int64_t(hkv) * D);
    const uint32_t kv_row_bytes = uint32_t(kv_stride) * 2u;
    // key base of step st, whose tile entry is ent (two 64-key steps per entry)
    auto kbase_at = [](int ent, int st) { return (ent >> 1) * kBlock + kStep * (st & 1); };
    auto issue_k = [&](int st, int kbase) {
        const uint64_t off = uint64_t(uint32_t(kbase)) * kv_row_bytes;
        T::load_async(ktile(st), reinterpret_cast<const bf16*>(Kh + off), kvs, wave, lane);
        // the keys' subtree ends ride with the K tile (wave w stages 16 of
        // them): a step's mask is applied while the step before it runs its
        // P V product, and reading LDS there issues no global load whose
        // wait would also drain the prefetch
        if (lane < 16) dma4(se + kbase + 16 * wave, 4u * lane, lds_addr(serow(st) + 64 * wave));
    };
    auto issue_v = [&](int st, int kbase) {
        const uint64_t off = uint64_t(uint32_t(kbase)) * kv_row_bytes;
        T::load_async(vtile(st), reinterpret_cast<const bf16*>(Vh + off), kvs, wave, lane);
    };
    // S^T = K Q^T (unscaled) of step st for its two 32-key blocks kk:
    // register r holds key kbase + 32 kk + 8 (r / 4) + 4 h + r % 4 against
    // this lane's query
    auto scores = [&](int st, f32x16 (&sc)[2]) {
        const lds_char* kt = ktile(st);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[kk][r] = 0.f;
#pragma unroll
            for (int x = 0; x < NX; ++x)
                sc[kk] = mfma32x32x16(T::frag_at(kt + 32 * kk * T::kRowBytes, roff[x]), qf[x], sc[kk]);
        }
    };
    // partial tiles: key <= qi and qi <= se[key], i.e.
    // 8 (r / 4) + r % 4 <= qi - (kbase + 32 kk + 4 h) and qi <= se[key]
    auto mask = [&](int st, int kbase, f32x16 (&s)[2]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int k0 = kbase + 32 * kk + 4 * h, lim = qi - k0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x4 sek = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
                    serow(st) + 4 * (32 * kk + 8 * j + 4 * h));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!(8 * j + i <= lim && qi <= sek[i])) s[kk][4 * j + i] = -INFINITY;
            }
        }
    };
    // Online softmax in base 2, one query per lane (its keys split over the
    // lane pair l, l ^ 32).  The running max m_run is kept in scaled units
    // and only moves when some lane's tile max exceeds it by more than
    // kRescaleSlack (log2 units): O and l are both relative to the same
    // reference, so a stale one changes nothing but the magnitude of p,
    // which stays <= 2^kRescaleSlack, and the O rescale runs a few times per
    // row instead of nearly every step.  rebase() takes the row max of a
    // step's masked scores, moves the reference if needed and returns the
    // factor alpha that carries sums over the old reference to the new one
    // (resc false: no move, alpha unused).  maximum (not maxnum) lowers to
    // v_maximum3_f32 with no NaN-quieting of the accumulator inputs.
    auto rebase = [&](float mx, bool ok, bool& resc) {
        const LanePair mp = lane_pair32(mx);
        mx = __builtin_elementwise_maximum(mp.lo, mp.hi);
        const float mt = mx * scale_log2;
        resc = __any(ok & (mt > m_run + kRescaleSlack));
        const float mnew = resc ? fmaxf(m_run, mt) : m_run;
        const float alpha = fast_exp2(m_run - (mnew == -INFINITY ? 0.f : mnew));
        m_run = mnew;
        return alpha;
    };
    auto max2 = [](float m, float a, float b) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, a), b);
    };

    f32x16 sa[2], sb[2];
    // The row's entries ride in scalar registers: a pair of steps (one
    // entry) holds its own entry and the next, and requests the one after,
    // so the steps never wait on a load of the list (one load per pair,
    // a pair ahead, instead of three per step at the point of use).
    const int nent = nsteps >> 1;
    int ent_c = nent > 0 ? row_ent[beg] : 0, ent_n = nent > 1 ? row_ent[beg + 1] : ent_c;
    if (nsteps > 0) {
        issue_k(0, kbase_at(ent_c, 0));
        issue_v(0, kbase_at(ent_c, 0));
        if (nsteps > 1) issue_k(1, kbase_at(ent_c, 1));
    }
#pragma unroll
    for (int x = 0; x < NX; ++x) consume(qf[x]);
    wait_vm_all();
    __syncthreads();
    if (nsteps > 0) {
        // step 0's scores, mask, reference and exp2 arguments; the steps
        // below prepare each following step the same way beside their P V
        scores(0, sa);
        if (ent_c & 1) mask(0, kbase_at(ent_c, 0), sa);
        float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            m0 = max2(m0, sa[0][r], sa[0][r + 1]);
            m1 = max2(m1, sa[1][r], sa[1][r + 1]);
        }
        bool resc;
        rebase(__builtin_elementwise_maximum(m0, m1), true, resc);  // O and l are still zero
        const float muse = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r) sa[kk][r] = __builtin_fmaf(sa[kk][r], scale_log2, -muse);
    }
    __syncthreads();  // every wave is done with K(0) and its subtree ends before K(2) replaces them

#define TREEATTN_SCHED() __builtin_amdgcn_sched_barrier(0)
    // One step.  On entry sc holds step st's exp2 arguments
    // (scale log2e S - m, masked entries -inf).  The scores of step st + 1
    // (independent of the exp work; after the last step they read a stale K
    // buffer and are discarded) run as two chains, one per 32-key block,
    // with this step's exponentials between their MFMAs; then O^T += V^T P^T
    // runs with the VALU work that prepares step st + 1 between its MFMAs:
    // this step's row sum, the next step's mask, row max and reference, and
    // its exp2 arguments.  Scheduling barriers pin that order, and every LDS
    // operand is read two MFMA groups before its use: left to itself the
    // compiler fed one score chain through a single register quadruple, so
    // each of its MFMAs waited a full LDS round trip, and it gathered the
    // row sum and the row max into one serial chain at the top of each step,
    // beside no MFMA at all.  Empty volatile asms hold each slot's results
    // in place: without them the row sum and the exp2 arguments were sunk
    // past the barriers to their uses.
    auto step = [&](int st, f32x16 (&sc)[2], f32x16 (&sn)[2], auto last_t) {
        constexpr bool kLast = decltype(last_t)::value;
        const bool has_next = !kLast;
        // the next step's entry: this pair's for an even st, the next pair's
        // for an odd one (equal to it, or unused, past the last step)
        const int ent1 = (st & 1) ? ent_n : ent_c;
        const bool next_partial = has_next && (ent1 & 1);
        if (st + 2 < nsteps) issue_k(st + 2, kbase_at(ent_n, st + 2));
        if (has_next) issue_v(st + 1, kbase_at(ent1, st + 1));
        const lds_char* vt = vtile(st);
        const lds_char* ktn = ktile(st + 1);
        auto rd_k = [&](int x, int kk) { return T::frag_at(ktn + 32 * kk * T::kRowBytes, roff[x]); };
        // A = 32 d x 16 keys of V^T, read transposed from the V tile in the
        // P^T key order (rows 16 m + 4 h + {0..3, 8..11}); unit u = NT m + t, so
        // consecutive MFMAs update different accumulators
        auto rd_v = [&](int u) {
            const int rb = 16 * (u / NT) * T::kRowBytes;
            return join_tr(T::tr_at(vt + rb, toff[u % NT][0]), T::tr_at(vt + rb, toff[u % NT][1]));
        };
        constexpr int kE = 32 / NX;  // exponentials per k-step
        bf16x8 kf[NX][2], va[4 * NT], pb[4];
        // p = exp2(argument), and the P^T operand of k-step m (keys
        // 16 m + {4 h + 0..3, 8 + 4 h + 0..3}) once its 8 are done
        auto ex = [&](int e) {
            const int kk = e >> 4, r = e & 15;
            sc[kk][r] = fast_exp2(sc[kk][r]);
            if ((e & 7) == 7) {
                const f32x16& a = sc[kk];
                const int b = 8 * ((e >> 3) & 1);
                pb[e >> 3] = to_bf16x8(f32x4{a[b], a[b + 1], a[b + 2], a[b + 3]},
                                       f32x4{a[b + 4], a[b + 5], a[b + 6], a[b + 7]});
            }
        };
        if constexpr (kLast) {
            // The last step has no next scores to compute.  Its keys come
            // after every query of a wave whose queries all precede them
            // (the second half of the diagonal tile for the first two
            // waves): every p is then exactly 0, and the wave skips the
            // exponentials and P V altogether.
            if (kbase_at(ent_c, st) <= qb * kBlock + 32 * wave + 31) {
#pragma unroll
                for (int e = 0; e < 32; ++e) ex(e);
#pragma unroll
                for (int u = 0; u < 4 * NT; ++u) va[u] = rd_v(u);
                float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 32; ++e) rs[e & 3] += sc[e >> 4][e & 15];
#pragma unroll
                for (int u = 0; u < 4 * NT; ++u) oacc[u % NT] = mfma32x32x16(va[u], pb[u / NT], oacc[u % NT]);
                l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
            }
            return;
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            kf[x][0] = rd_k(x, 0);
            kf[x][1] = rd_k(x, 1);
        }
        TREEATTN_SCHED();
#pragma unroll
        for (int x = 0; x < NX; ++x) {
            if (x + 2 < NX) {
                kf[x + 2][0] = rd_k(x + 2, 0);
                kf[x + 2][1] = rd_k(x + 2, 1);
            } else {
                va[x + 2 - NX] = rd_v(x + 2 - NX);
            }
            sn[0] = mfma32x32x16(kf[x][0], qf[x], x == 0 ? f32x16{} : sn[0]);
#pragma unroll
            for (int e = 0; e < kE / 2; ++e) ex(kE * x + e);
            sn[1] = mfma32x32x16(kf[x][1], qf[x], x == 0 ? f32x16{} : sn[1]);
#pragma unroll
            for (int e = kE / 2; e < kE; ++e) ex(kE * x + e);
            TREEATTN_SCHED();
        }

        // P V: the first quarter of its MFMAs carries the row sum (four
        // partial sums), then the next step's mask (partial tiles), the
        // second quarter its row max (two chains), and the second half the
        // reference move and the exp2 arguments
        constexpr int U = 4 * NT, UA = U / 4, UC = U / 2;
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
        float m0 = -INFINITY, m1 = -INFINITY, alpha = 1.f, muse = 0.f;
        bool resc = false;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u + 2 < U) va[u + 2] = rd_v(u + 2);
            oacc[u % NT] = mfma32x32x16(va[u], pb[u / NT], oacc[u % NT]);
            if (u < UA) {
                constexpr int n = 32 / UA;
#pragma unroll
                for (int i = 0; i < n; ++i) {
                    const int e = n * u + i;
                    rs[e & 3] += sc[e >> 4][e & 15];
                }
                asm volatile("" : "+v"(rs[0]), "+v"(rs[1]), "+v"(rs[2]), "+v"(rs[3]));
            } else if (u < UC) {
                constexpr int n = 16 / (UC - UA);  // per chain
#pragma unroll
                for (int i = 0; i < n; i += 2) {
                    const int r = n * (u - UA) + i;
                    m0 = max2(m0, sn[0][r], sn[0][r + 1]);
                    m1 = max2(m1, sn[1][r], sn[1][r + 1]);
                }
                asm volatile("" : "+v"(m0), "+v"(m1));
            } else {
                if (u == UC) {
                    alpha = rebase(__builtin_elementwise_maximum(m0, m1), has_next, resc);
                    muse = m_run == -INFINITY ? 0.f : m_run;
                }
                constexpr int n = 32 / (U - UC);
#pragma unroll
                for (int i = 0; i < n; ++i) {
                    const int e = n * (u - UC) + i;
                    float a = __builtin_fmaf(sn[e >> 4][e & 15], scale_log2, -muse);
                    asm volatile("" : "+v"(a));
                    sn[e >> 4][e & 15] = a;
                }
            }
            TREEATTN_SCHED();
            if (u == UA - 1 && next_partial) mask(st + 1, kbase_at(ent1, st + 1), sn);
        }
        l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        if (resc) {
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t) oacc[t] *= alpha;
        }

        wait_vm_all();
        __syncthreads();
    };
    // a query block's step count is even (two per 128-key tile), so the
    // score buffers alternate without copies
    for (int st = 0; st + 2 < nsteps; st += 2) {
        const int ent_nn = row_ent[beg + min((st >> 1) + 2, nent - 1)];
        step(st, sa, sb, std::false_type{});
        step(st + 1, sb, sa, std::false_type{});
        ent_c = ent_n;
        ent_n = ent_nn;
    }
    if (nsteps > 0) {
        step(nsteps - 2, sa, sb, std::false_type{});
        step(nsteps - 1, sb, sa, std::true_type{});
    }

#undef TREEATTN_SCHED

    // epilogue: normalise, write O (bf16) and LSE (natural log)
    const LanePair lp = lane_pair32(l_run);
    float l = lp.lo + lp.hi;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* orow = O + int64_t(qi) * q_stride + int64_t(h_q) * D + 4 * h;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x16& a = oacc[t];
            st8(orow + 32 * t + 8 * j, u32x2{pack_bf16x2(a[4 * j] * inv, a[4 * j + 1] * inv),
                                             pack_bf16x2(a[4 * j + 2] * inv, a[4 * j + 3] * inv)});
        }
    if (h == 0) LSE[int64_t(h_q) * L + qi] = l > 0.f ? (m_run + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int32_t* se, const MetaPtrs& mp, const AttnShape& sh,
                           hipStream_t stream, const RowSel& sel, const RopeArgs& rope) {
    // the work items are (query block of the list, query head)
    const int32_t* q_order = sel.q_list ? sel.q_list : mp.q_order;
    const unsigned n_q = sel.q_list ? unsigned(sel.n_q) : unsigned(sh.nb);
    if (n_q == 0) return hipSuccess;
    const dim3 grid(n_q * unsigned(sh.Hq));
    const float sl2 = sh.scale * 1.4426950408889634f;
    const auto* Q = static_cast<const bf16*>(q);
    const auto* K = static_cast<const bf16*>(k);
    const auto* V = static_cast<const bf16*>(v);
    auto* O = static_cast<bf16*>(o);
    auto* Qr = static_cast<bf16*>(rope.q_rot);
    if (sh.D == 128 && rope.tab)
        fwd_bf16_kernel<128, true><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, q_order, mp.row_ptr,
                                                                   mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2,
                                                                   rope.pos, rope.tab, Qr);
    else if (sh.D == 128)
        fwd_bf16_kernel<128, false><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, q_order, mp.row_ptr,
                                                                    mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2,
                                                                    nullptr, nullptr, nullptr);
    else if (sh.D == 64 && rope.tab)
        fwd_bf16_kernel<64, true><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, q_order, mp.row_ptr,
                                                                  mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2,
                                                                  rope.pos, rope.tab, Qr);
    else if (sh.D == 64)
        fwd_bf16_kernel<64, false><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, q_order, mp.row_ptr,
                                                                   mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2,
                                                                   nullptr, nullptr, nullptr);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace treeattn
