"""The C ABI from C: a C99 program compiled with gcc against
include/tree_attn.h (no C++ and no HIP headers) and linked to
libtreeattn.so packs the tree-training guide's worked example and checks
it against the hand-derived golden file, then exercises the error path.
Host-only calls, so it runs without a GPU."""

import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "prefix_tree_attention_amd")
GOLDEN = os.path.join(ROOT, "tests", "golden", "worked_example.json")

C_SOURCE = r"""
#include <stdio.h>
#include "tree_attn.h"

int main(void) {
    /* Seq0 [A,B,C,D], Seq1 [A,B,E,F], Seq2 [A,G,H] with A..H = 1..8 */
    const int32_t ids[12] = {1, 2, 3, 4, 1, 2, 5, 6, 1, 7, 8, 0};
    const uint8_t mask[12] = {1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 0};
    tree_pack_t* p = NULL;
    int rc = tree_pack(ids, mask, 3, 4, 128, TREE_BLOCK, 0, 0, &p);
    if (rc != TREE_OK) {
        printf("pack failed %d %s\n", rc, tree_last_error());
        return 1;
    }
    tree_trie_view v;
    tree_pack_stats_t s;
    if (tree_pack_trie(p, 0, &v) != TREE_OK || tree_pack_stats(p, &s) != TREE_OK) return 2;
    printf("abi %d tries %lld n %lld L %lld nodes %lld seqs %lld\n", tree_abi_version(),
           (long long)tree_pack_num_tries(p), (long long)v.n_tokens, (long long)v.L, (long long)v.n_nodes,
           (long long)v.n_seqs);
    printf("ids");
    for (int i = 0; i < 8; ++i) printf(" %d", v.token_ids[i]);
    printf("\nse");
    for (int i = 0; i < 8; ++i) printf(" %d", v.subtree_end[i]);
    printf("\npairs %lld unpacked %lld tree %lld original %lld\n", (long long)s.n_pairs,
           (long long)s.unpacked_pairs, (long long)s.tree_tokens, (long long)s.original_tokens);
    tree_pack_free(p);
    p = NULL;
    rc = tree_pack(ids, mask, 3, 4, 100, TREE_BLOCK, 0, 0, &p); /* not a multiple of 128 */
    printf("misaligned %d %s\n", rc, p == NULL ? "null" : "set");
    return 0;
}
"""


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = os.path.join(LIBDIR, "libtreeattn.so")
    if not os.path.exists(lib):
        pytest.skip("libtreeattn.so is not built")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "pack_example.c"
    src.write_text(C_SOURCE)
    out = d / "pack_example"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(out), "-L", LIBDIR, "-ltreeattn", f"-Wl,-rpath,{LIBDIR}"], check=True)
    return str(out)


def test_c_program_packs_the_worked_example(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    g = json.load(open(GOLDEN))
    assert lines[0] == f"abi 7 tries 1 n {g['n_tokens']} L {g['L']} nodes {len(g['node_start'])} seqs 3"
    assert lines[1] == "ids " + " ".join(map(str, g["token_ids_real"]))
    assert lines[2] == "se " + " ".join(map(str, g["subtree_end_real"]))
    assert lines[3] == "pairs 22 unpacked 26 tree 8 original 11"
    assert lines[4] == "misaligned -2 null"  # TREE_E_ALIGN, *out left NULL
