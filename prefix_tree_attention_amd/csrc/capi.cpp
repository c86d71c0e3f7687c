// C ABI of libtreeattn: argument validation and dispatch to the device
// launchers.  See include/tree_attn.h for the contract.

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "device.h"
#include "status.h"

namespace treeattn {

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_L(int64_t L, const char* fn) {
    if (L <= 0 || L % kBlock != 0 || L > kMaxL)
        return set_error(TREE_E_ARG, "%s: L=%lld must be a positive multiple of %d and <= %lld", fn,
                         (long long)L, kBlock, (long long)kMaxL);
    return TREE_OK;
}

}  // namespace

int check_attn(const char* fn, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t dtype) {
    if (int rc = check_L(L, fn)) return rc;
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq > 4096)
        return set_error(TREE_E_ARG, "%s: bad head counts Hq=%d Hkv=%d (need Hq %% Hkv == 0)", fn, Hq, Hkv);
    if (L * int64_t(Hq) >= (int64_t(1) << 31))
        return set_error(TREE_E_ARG, "%s: L * Hq = %lld rows exceeds 2^31 - 1", fn, (long long)(L * int64_t(Hq)));
    if (dtype == TREE_DTYPE_BF16) {
        if (D != 64 && D != 128) return set_error(TREE_E_ARG, "%s: bf16 path supports D in {64,128}, got %d", fn, D);
    } else if (dtype == TREE_DTYPE_FP32) {
        if (D != 32 && D != 64 && D != 128)
            return set_error(TREE_E_ARG, "%s: fp32 path supports D in {32,64,128}, got %d", fn, D);
    } else {
        return set_error(TREE_E_ARG, "%s: unknown dtype %d", fn, dtype);
    }
    if (!std::isfinite(scale) || !(scale > 0.f))
        return set_error(TREE_E_ARG, "%s: scale must be finite and positive", fn);
    return TREE_OK;
}

namespace {

int hip_status(hipError_t e, const char* fn) {
    if (e != hipSuccess) return set_error(TREE_E_HIP, "%s: HIP error %d (%s)", fn, int(e), hipGetErrorString(e));
    clear_error();
    return TREE_OK;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// the gather of tree_gather_logprobs and tree_gather_logprobs_rows
int gather_logprobs(const char* name, const void* logits, int64_t row0, int64_t n_rows, int64_t L, int64_t V,
                    int32_t dtype, const float* d_lse, const float* d_ent, const int32_t* d_ids,
                    const int32_t* d_row_pos, int64_t B, int64_t S, float pad_value, float* d_logp, float* d_out_ent,
                    void* stream) {
    if (L < 0 || L > (int64_t(1) << 31) - 1 || V <= 0 || V > (int64_t(1) << 31) - 1 || B < 0 || S < 0 ||
        (S > 0 && B > ((int64_t(1) << 40) / S)))
        return set_error(TREE_E_ARG, "%s: bad shape L=%lld V=%lld B=%lld S=%lld", name, (long long)L, (long long)V,
                         (long long)B, (long long)S);
    if (row0 < 0 || n_rows < 0 || row0 > L - n_rows)
        return set_error(TREE_E_ARG, "%s: rows [%lld, %lld) outside [0, %lld)", name, (long long)row0,
                         (long long)(row0 + n_rows), (long long)L);
    if (dtype != TREE_DTYPE_BF16 && dtype != TREE_DTYPE_FP32)
        return set_error(TREE_E_ARG, "%s: unknown dtype %d", name, dtype);
    if (B * S == 0) {
        clear_error();
        return TREE_OK;
    }
    if (!d_row_pos || !d_logp || !d_out_ent || (L > 0 && (!d_lse || !d_ent || !d_ids)) || (n_rows > 0 && !logits))
        return set_error(TREE_E_ARG, "%s: NULL device pointer", name);
    return hip_status(launch_gather_logprobs(logits, row0, n_rows, L, V, dtype, d_lse, d_ent, d_ids, d_row_pos, B, S,
                                             pad_value, d_logp, d_out_ent, static_cast<hipStream_t>(stream)),
                      name);
}

}  // namespace
}  // namespace treeattn

using namespace treeattn;

extern "C" {

int tree_abi_version(void) { return TREE_ATTN_ABI_VERSION; }

size_t tree_meta_workspace_bytes(int64_t L) {
    if (L <= 0 || L % kBlock != 0 || L > kMaxL) return 0;
    return size_t(meta_layout(L).words) * sizeof(int32_t);
}

int tree_meta(const int32_t* d_se, int64_t L, int32_t* d_pos, uint8_t* d_tile_class, void* d_ws,
              size_t ws_bytes, void* stream) {
    if (int rc = check_L(L, "tree_meta")) return rc;
    if (!d_se || !d_pos || !d_tile_class || !d_ws) return set_error(TREE_E_ARG, "tree_meta: NULL device pointer");
    if (!aligned16(d_se) || !aligned16(d_ws))
        return set_error(TREE_E_ARG, "tree_meta: d_se and d_ws must be 16-byte aligned");
    if (ws_bytes < tree_meta_workspace_bytes(L))
        return set_error(TREE_E_WORKSPACE, "tree_meta: workspace %zu < %zu bytes", ws_bytes,
                         tree_meta_workspace_bytes(L));
    return hip_status(launch_meta(d_se, L, d_pos, d_tile_class, d_ws, static_cast<hipStream_t>(stream)),
                      "tree_meta");
}

int tree_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* d_se,
                  const void* d_meta_ws, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t dtype,
                  void* stream) {
    if (int rc = check_attn("tree_attn_fwd", L, Hq, Hkv, D, scale, dtype)) return rc;
    if (!q || !k || !v || !o || !lse || !d_se || !d_meta_ws)
        return set_error(TREE_E_ARG, "tree_attn_fwd: NULL device pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_se) ||
        !aligned16(d_meta_ws))
        return set_error(TREE_E_ARG, "tree_attn_fwd: tensors must be 16-byte aligned");
    const AttnShape sh{L, int(L / kBlock), Hq, Hkv, D, scale};
    const MetaPtrs mp = meta_ptrs(d_meta_ws, L);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == TREE_DTYPE_BF16)
        e = launch_fwd_bf16(q, k, v, o, lse, d_se, mp, sh, s);
    else
        e = launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                           static_cast<float*>(o), lse, d_se, mp, sh, s);
    return hip_status(e, "tree_attn_fwd");
}

size_t tree_attn_bwd_workspace_bytes(int64_t L, int32_t Hq, int32_t D, int32_t dtype) {
    (void)D;
    (void)dtype;
    if (L <= 0 || Hq <= 0) return 0;
    return round256(2 * size_t(L) * size_t(Hq) * sizeof(float));  // Delta [Hq, L], LSE log2 e [Hq, L]
}

int tree_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, const int32_t* d_se, const void* d_meta_ws, void* d_ws,
                  size_t ws_bytes, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t dtype,
                  void* stream) {
    return tree_attn_bwd_phase(TREE_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, d_se, d_meta_ws, d_ws, ws_bytes, L,
                               Hq, Hkv, D, scale, dtype, stream);
}

int tree_attn_bwd_phase(int32_t phase, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv, const int32_t* d_se,
                        const void* d_meta_ws, void* d_ws, size_t ws_bytes, int64_t L, int32_t Hq, int32_t Hkv,
                        int32_t D, float scale, int32_t dtype, void* stream) {
    if (phase < TREE_BWD_ALL || phase > TREE_BWD_DQ_DELTA)
        return set_error(TREE_E_ARG, "tree_attn_bwd: unknown phase %d", phase);
    if (int rc = check_attn("tree_attn_bwd", L, Hq, Hkv, D, scale, dtype)) return rc;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !d_se || !d_meta_ws || !d_ws)
        return set_error(TREE_E_ARG, "tree_attn_bwd: NULL device pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse) || !aligned16(d_se) ||
        !aligned16(d_meta_ws) || !aligned16(d_ws))
        return set_error(TREE_E_ARG, "tree_attn_bwd: tensors must be 16-byte aligned");
    const size_t need = tree_attn_bwd_workspace_bytes(L, Hq, D, dtype);
    if (ws_bytes < need)
        return set_error(TREE_E_WORKSPACE, "tree_attn_bwd: workspace %zu < %zu bytes", ws_bytes, need);
    const AttnShape sh{L, int(L / kBlock), Hq, Hkv, D, scale};
    const MetaPtrs mp = meta_ptrs(d_meta_ws, L);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* delta = static_cast<float*>(d_ws);
    hipError_t e;
    if (dtype == TREE_DTYPE_BF16)
        e = launch_bwd_bf16(phase, q, k, v, o, lse, dout, dq, dk, dv, d_se, mp, delta, sh, s);
    else
        e = launch_bwd_f32(phase, static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), static_cast<const float*>(o), lse,
                           static_cast<const float*>(dout), static_cast<float*>(dq), static_cast<float*>(dk),
                           static_cast<float*>(dv), d_se, mp, delta, sh, s);
    return hip_status(e, "tree_attn_bwd");
}

size_t tree_rope_table_bytes(int64_t P, int32_t D) {
    if (P <= 0 || P > kMaxL || D <= 0 || D % 16 != 0 || D > 4096) return 0;
    return round256(size_t(P) * size_t(D / 2) * 2 * sizeof(float));
}

int tree_rope_table(double base, int64_t P, int32_t D, float* d_tab, size_t tab_bytes, void* stream) {
    const size_t need = tree_rope_table_bytes(P, D);
    if (need == 0) return set_error(TREE_E_ARG, "tree_rope_table: bad P=%lld or D=%d", (long long)P, D);
    if (!std::isfinite(base) || !(base > 1.0)) return set_error(TREE_E_ARG, "tree_rope_table: base must be > 1");
    if (!d_tab || !aligned16(d_tab)) return set_error(TREE_E_ARG, "tree_rope_table: NULL or misaligned table");
    if (tab_bytes < need) return set_error(TREE_E_WORKSPACE, "tree_rope_table: %zu < %zu bytes", tab_bytes, need);
    return hip_status(launch_rope_table(d_tab, P, D, base, static_cast<hipStream_t>(stream)), "tree_rope_table");
}

int tree_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse, void* q_rot, void* k_rot,
                       const int32_t* d_pos, const float* d_tab, size_t tab_bytes, const int32_t* d_se,
                       const void* d_meta_ws, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                       void* stream) {
    if (int rc = check_attn("tree_attn_fwd_rope", L, Hq, Hkv, D, scale, TREE_DTYPE_BF16)) return rc;
    if (!q || !k || !v || !o || !lse || !q_rot || !k_rot || !d_pos || !d_tab || !d_se || !d_meta_ws)
        return set_error(TREE_E_ARG, "tree_attn_fwd_rope: NULL device pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(q_rot) || !aligned16(k_rot) ||
        !aligned16(d_tab) || !aligned16(d_se) || !aligned16(d_meta_ws))
        return set_error(TREE_E_ARG, "tree_attn_fwd_rope: tensors must be 16-byte aligned");
    if (tab_bytes < tree_rope_table_bytes(L, D))
        return set_error(TREE_E_WORKSPACE, "tree_attn_fwd_rope: the table must cover positions 0 .. L - 1");
    const AttnShape sh{L, int(L / kBlock), Hq, Hkv, D, scale};
    const MetaPtrs mp = meta_ptrs(d_meta_ws, L);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_rope_tab(k, k_rot, d_pos, d_tab, L, Hkv, D, s);
    RopeArgs rope;
    rope.pos = d_pos;
    rope.tab = d_tab;
    rope.q_rot = q_rot;
    if (e == hipSuccess) e = launch_fwd_bf16(q, k_rot, v, o, lse, d_se, mp, sh, s, RowSel(), rope);
    return hip_status(e, "tree_attn_fwd_rope");
}

int tree_attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, const int32_t* d_pos, const float* d_tab,
                       size_t tab_bytes, const int32_t* d_se, const void* d_meta_ws, void* d_ws, size_t ws_bytes,
                       int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, void* stream) {
    if (int rc = check_attn("tree_attn_bwd_rope", L, Hq, Hkv, D, scale, TREE_DTYPE_BF16)) return rc;
    if (!q_rot || !k_rot || !v || !o || !lse || !dout || !dq || !dk || !dv || !d_pos || !d_tab || !d_se ||
        !d_meta_ws || !d_ws)
        return set_error(TREE_E_ARG, "tree_attn_bwd_rope: NULL device pointer");
    if (!aligned16(q_rot) || !aligned16(k_rot) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse) || !aligned16(d_tab) ||
        !aligned16(d_se) || !aligned16(d_meta_ws) || !aligned16(d_ws))
        return set_error(TREE_E_ARG, "tree_attn_bwd_rope: tensors must be 16-byte aligned");
    if (tab_bytes < tree_rope_table_bytes(L, D))
        return set_error(TREE_E_WORKSPACE, "tree_attn_bwd_rope: the table must cover positions 0 .. L - 1");
    const size_t need = tree_attn_bwd_workspace_bytes(L, Hq, D, TREE_DTYPE_BF16);
    if (ws_bytes < need)
        return set_error(TREE_E_WORKSPACE, "tree_attn_bwd_rope: workspace %zu < %zu bytes", ws_bytes, need);
    const AttnShape sh{L, int(L / kBlock), Hq, Hkv, D, scale};
    const MetaPtrs mp = meta_ptrs(d_meta_ws, L);
    RopeArgs rope;
    rope.pos = d_pos;
    rope.tab = d_tab;
    return hip_status(launch_bwd_bf16(kPhaseAll, q_rot, k_rot, v, o, lse, dout, dq, dk, dv, d_se, mp,
                                      static_cast<float*>(d_ws), sh, static_cast<hipStream_t>(stream), RowSel(),
                                      rope),
                      "tree_attn_bwd_rope");
}

int tree_logits_stats(const void* logits, int64_t L, int64_t V, int32_t dtype, float* d_lse, float* d_ent,
                      void* stream) {
    if (L < 0 || L > (int64_t(1) << 31) - 1 || V <= 0 || V > (int64_t(1) << 31) - 1)
        return set_error(TREE_E_ARG, "tree_logits_stats: bad shape L=%lld V=%lld", (long long)L, (long long)V);
    if (dtype != TREE_DTYPE_BF16 && dtype != TREE_DTYPE_FP32)
        return set_error(TREE_E_ARG, "tree_logits_stats: unknown dtype %d", dtype);
    if (L == 0) {
        clear_error();
        return TREE_OK;
    }
    if (!logits || !d_lse || !d_ent) return set_error(TREE_E_ARG, "tree_logits_stats: NULL device pointer");
    if ((reinterpret_cast<uintptr_t>(logits) & (dtype == TREE_DTYPE_BF16 ? 1u : 3u)) != 0)
        return set_error(TREE_E_ARG, "tree_logits_stats: logits not aligned to their element size");
    return hip_status(launch_logits_stats(logits, L, V, dtype, d_lse, d_ent, static_cast<hipStream_t>(stream)),
                      "tree_logits_stats");
}

int tree_gather_logprobs(const void* logits, int64_t L, int64_t V, int32_t dtype, const float* d_lse,
                         const float* d_ent, const int32_t* d_ids, const int32_t* d_row_pos, int64_t B, int64_t S,
                         float pad_value, float* d_logp, float* d_out_ent, void* stream) {
    return gather_logprobs("tree_gather_logprobs", logits, 0, L, L, V, dtype, d_lse, d_ent, d_ids, d_row_pos, B, S,
                           pad_value, d_logp, d_out_ent, stream);
}

int tree_gather_logprobs_rows(const void* logits_rows, int64_t row0, int64_t n_rows, int64_t L, int64_t V,
                              int32_t dtype, const float* d_lse, const float* d_ent, const int32_t* d_ids,
                              const int32_t* d_row_pos, int64_t B, int64_t S, float pad_value, float* d_logp,
                              float* d_out_ent, void* stream) {
    return gather_logprobs("tree_gather_logprobs_rows", logits_rows, row0, n_rows, L, V, dtype, d_lse, d_ent, d_ids,
                           d_row_pos, B, S, pad_value, d_logp, d_out_ent, stream);
}

int tree_rope(const void* x, void* y, const int32_t* d_pos, int64_t L, int32_t H, int32_t D, double base,
              int32_t inverse, int32_t dtype, void* stream) {
    if (L < 0 || L > (int64_t(1) << 31) - 1 || H <= 0 || D <= 0 || D % 2 != 0 || D > 4096 ||
        int64_t(H) * D > (int64_t(1) << 20))
        return set_error(TREE_E_ARG, "tree_rope: bad shape L=%lld H=%d D=%d (D even)", (long long)L, H, D);
    if (!std::isfinite(base) || !(base > 1.0)) return set_error(TREE_E_ARG, "tree_rope: base must be finite and > 1");
    if (dtype != TREE_DTYPE_BF16 && dtype != TREE_DTYPE_FP32)
        return set_error(TREE_E_ARG, "tree_rope: unknown dtype %d", dtype);
    if (L == 0) {
        clear_error();
        return TREE_OK;
    }
    if (!x || !y || !d_pos) return set_error(TREE_E_ARG, "tree_rope: NULL device pointer");
    const uintptr_t al = dtype == TREE_DTYPE_BF16 ? 1u : 3u;
    if ((reinterpret_cast<uintptr_t>(x) & al) || (reinterpret_cast<uintptr_t>(y) & al))
        return set_error(TREE_E_ARG, "tree_rope: tensors not aligned to their element size");
    return hip_status(launch_rope(x, y, d_pos, L, H, D, base, inverse ? 1 : 0, dtype, static_cast<hipStream_t>(stream)),
                      "tree_rope");
}

}  // extern "C"
