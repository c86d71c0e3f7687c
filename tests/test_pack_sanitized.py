"""The host packer built with AddressSanitizer and UBSan (CPU only).

pack.cpp and the error state (status.cpp) need no HIP runtime, so they are
compiled here with g++ -fsanitize=address,undefined into a small driver
that packs each batch through the C ABI (tree_pack_ordered, the views,
tree_pack_stats, tree_pack_concat / _concat_ids / _row_positions,
tree_partition) and writes every result to a file.  Any out-of-bounds
access, use after free, leak or undefined behaviour aborts the driver; its
outputs must equal the library's, byte for byte, on the configurations'
batches, two sweep points, random batches with non-contiguous masks and the
validation errors."""

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import workloads
import prefix_tree_attention_amd as pta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_tree_attention_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "tree_attn.h"

static void w64(FILE* f, int64_t x) { fwrite(&x, 8, 1, f); }
static void warr(FILE* f, const int32_t* p, int64_t n) { w64(f, n); if (n) fwrite(p, 4, size_t(n), f); }

int main(int argc, char** argv) {
    FILE* in = fopen(argv[1], "rb");
    FILE* out = fopen(argv[2], "wb");
    int64_t hdr[4];  // B, S, M, order
    if (fread(hdr, 8, 4, in) != 4) return 2;
    const int64_t B = hdr[0], S = hdr[1];
    std::vector<int32_t> ids(static_cast<size_t>(B * S));
    std::vector<uint8_t> mask(static_cast<size_t>(B * S));
    if (B * S && (fread(ids.data(), 4, ids.size(), in) != ids.size() ||
                  fread(mask.data(), 1, mask.size(), in) != mask.size())) return 2;
    fclose(in);
    tree_pack_t* p = nullptr;
    const int rc = tree_pack_ordered(ids.data(), mask.data(), B, S, hdr[2], TREE_BLOCK, 0, 0, int32_t(hdr[3]), &p);
    w64(out, rc);
    if (rc == TREE_OK) {
        const int64_t nt = tree_pack_num_tries(p);
        w64(out, nt);
        for (int64_t t = 0; t < nt; ++t) {
            tree_trie_view v;
            tree_pack_trie(p, t, &v);
            w64(out, v.n_tokens);
            w64(out, v.L);
            warr(out, v.token_ids, v.L);
            warr(out, v.node_id, v.L);
            warr(out, v.subtree_end, v.L);
            warr(out, v.node_start, v.n_nodes);
            warr(out, v.node_end, v.n_nodes);
            warr(out, v.node_parent, v.n_nodes);
            warr(out, v.seq_ids, v.n_seqs);
            warr(out, v.seq_iv_ptr, v.n_seqs + 1);
            warr(out, v.seq_iv, 2 * int64_t(v.seq_iv_ptr[v.n_seqs]));
        }
        tree_pack_stats_t s;
        tree_pack_stats(p, &s);
        w64(out, s.tree_tokens);
        w64(out, s.n_pairs);
        w64(out, s.unpacked_pairs);
        w64(out, s.tiles_full);
        w64(out, s.tiles_partial);
        w64(out, s.tiles_causal);
        int64_t total = 0;
        tree_pack_concat(p, nullptr, 0, &total);
        std::vector<int32_t> se(static_cast<size_t>(total)), cid(static_cast<size_t>(total)),
            rp(static_cast<size_t>(B * S));
        tree_pack_concat(p, se.data(), total, &total);
        tree_pack_concat_ids(p, cid.data(), total);
        tree_pack_row_positions(p, rp.data(), B * S);
        warr(out, se.data(), total);
        warr(out, cid.data(), total);
        warr(out, rp.data(), B * S);
        tree_pack_free(p);
    }
    std::vector<int32_t> grp(static_cast<size_t>(B > 0 ? B : 1));
    int64_t tau = 0;
    std::vector<int64_t> costs(4);
    const int prc = tree_partition(ids.data(), mask.data(), B, S, 4, grp.data(), &tau, costs.data());
    w64(out, prc);
    if (prc == TREE_OK) {
        warr(out, grp.data(), B);
        w64(out, tau);
        for (int64_t c : costs) w64(out, c);
    }
    fclose(out);
    return 0;
}
"""


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("asan")
    drv = d / "driver.cpp"
    drv.write_text(DRIVER)
    exe = d / "pack_asan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "status.cpp"), str(drv), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("sanitized build failed:\n" + r.stderr[-4000:])
    return d, str(exe)


def _run_sanitized(sanitized, ids, mask, M, order):
    d, exe = sanitized
    ids = np.ascontiguousarray(ids, np.int32)
    mask = np.ascontiguousarray(mask, np.uint8)
    fin, fout = d / "in.bin", d / "out.bin"
    with open(fin, "wb") as f:
        f.write(struct.pack("<4q", ids.shape[0], ids.shape[1], M, order))
        f.write(ids.tobytes())
        f.write(mask.tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, "sanitizer report:\n" + (r.stderr[-4000:] or r.stdout[-4000:])
    return fout.read_bytes()


def _expected(ids, mask, M, order):
    """The same records, from the library through ctypes."""
    out = bytearray()
    w = lambda x: out.extend(struct.pack("<q", int(x)))  # noqa: E731

    def arr(a):
        a = np.ascontiguousarray(a, np.int32)
        w(a.size)
        out.extend(a.tobytes())

    try:
        tries, st = pta.pack(ids, mask, M, order=("ffd", "prefix")[order])
        rc = 0
    except pta.TreeAttnError as e:
        rc = e.code
    w(rc)
    if rc == 0:
        w(len(tries))
        for t in tries:
            w(t.n_tokens)
            w(t.L)
            for a in (t.token_ids, t.node_id, t.subtree_end, t.node_start, t.node_end, t.node_parent, t.seq_ids,
                      t.seq_iv_ptr, t.seq_iv.reshape(-1)):
                arr(a)
        for k in ("tree_tokens", "n_pairs", "unpacked_pairs", "tiles_full", "tiles_partial", "tiles_causal"):
            w(st[k])
        se, tok, rp, _, _ = pta.pack_batch(ids, mask, M, order=("ffd", "prefix")[order])
        arr(se)
        arr(tok)
        arr(rp.reshape(-1))
    try:
        grp, tau, costs = pta.partition(ids, mask, 4)
        w(0)
        arr(grp)
        w(tau)
        for c in costs:
            w(c)
    except pta.TreeAttnError as e:
        w(e.code)
    return bytes(out)


def _batches():
    for c in ("1", "2", "3", "4a", "4b"):
        w = workloads.make_workload(c)
        yield f"config{c}", w.ids, w.mask, w.max_tokens_per_mb
    for L_, b in ((8192, 8), (16384, 2)):
        w = workloads.sweep_workload(L_, b)
        yield f"sweep{L_}-{b}", w.ids, w.mask, w.max_tokens_per_mb
    rng = np.random.default_rng(99)
    for s in range(8):
        seqs = []
        for _ in range(int(rng.integers(1, 20))):
            if seqs and rng.random() < 0.6:
                base = seqs[int(rng.integers(len(seqs)))]
                cut = int(rng.integers(1, len(base) + 1))
                seqs.append(np.concatenate([base[:cut], rng.integers(0, 4, int(rng.integers(1, 60)))]).astype(np.int32))
            else:
                seqs.append(rng.integers(0, 4, int(rng.integers(1, 90))).astype(np.int32))
        ids, mask = workloads.pad_rows(seqs)
        # non-contiguous masks: shift a few rows' tokens right, leaving holes
        ids2 = np.zeros((ids.shape[0], ids.shape[1] + 5), np.int32)
        mask2 = np.zeros_like(ids2, np.uint8)
        for r in range(ids.shape[0]):
            n = int(mask[r].sum())
            cols = np.sort(rng.choice(ids2.shape[1], n, replace=False))
            ids2[r, cols] = ids[r, :n]
            mask2[r, cols] = 1
        yield f"random{s}", ids2, mask2, 256
    ids, mask = workloads.worked_example()
    bad = mask.copy()
    bad[1] = 0
    yield "empty-row", ids, bad, 128
    yield "too-long", ids, mask, 0


@pytest.mark.parametrize("order", [0, 1])
def test_sanitized_packer_matches_library(sanitized, order):
    for name, ids, mask, M in _batches():
        got = _run_sanitized(sanitized, ids, mask, M, order)
        assert got == _expected(ids, mask, M, order), f"{name}: sanitized packer output differs"
