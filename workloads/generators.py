"""Synthetic rollout batches shaped like the pages' workloads.

The pages measure on the tau2 / tau^2-bench agent task (Qwen3-8B,
n_samples 8, responses up to 8192 tokens, 32768 tokens per micro-batch) and
on GRPO-style groups of samples per prompt.  Neither the data set nor the
weights exist here, so these generators stand in for their *shapes*: token
ids are uniform random, which means two rollouts share a prefix exactly
where the generator makes them share one.

Every generator is seeded and deterministic.  Batches come out in the
padded tensor-dict form ``ids[B, S]`` int32 plus ``mask[B, S]`` uint8, real
tokens left-aligned in each row.

Configurations:
  1  tiny: 2 prompts x 48 tokens, 4 responses each of U[16,64] tokens; in
     prompt 0, response 3 repeats the first m tokens of response 0
     (m ~ U[1, min(len0, len3) - 1]) and then differs.  V = 1000.
     M = 512; 1 head, D = 64, fp32, forward only.
  2  GRPO: 16 prompts U[256,1024] x 8 responses U[128,2048], V = 151936.
     M = 8192; 32q/8kv heads, D = 128, bf16.
  3  multi-turn agentic: one 2048-token system prefix common to every
     sample; 4 prompt groups of 8 samples; for each of 4 turns a group of
     two or more samples splits into two halves with probability 0.5 (each
     half gets its own turn text), else the group shares one turn text;
     turns are U[256,1024] tokens; then every sample ends with its own
     response of U[256,8192] tokens.  M = 32768.
  4a deep-shared: one 16384-token prefix + 64 leaves x 256 tokens, leaf
     first tokens distinct.  M = 32768.
  4b no sharing: 16 disjoint sequences x 2048 tokens, distinct first
     tokens.  M = 32768.
  5  sweep: the config-2 generator with b samples per prompt and
     M = L in {8192, 16384, 32768, 65536}; ceil(4L / (640 + 1088 b))
     prompts, i.e. about four full tries.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

VOCAB_BIG = 151936

CONFIG_NAMES = {
    "1": "tiny-fwd",
    "2": "grpo-16x8",
    "3": "multiturn-agentic",
    "4a": "deep-shared-16k+64x256",
    "4b": "no-sharing-16x2048",
}


@dataclass
class Workload:
    name: str
    config: str
    ids: np.ndarray          # int32 [B, S]
    mask: np.ndarray         # uint8 [B, S]
    max_tokens_per_mb: int
    hq: int
    hkv: int
    d: int
    dtype: str               # "fp32" | "bf16"
    backward: bool
    qkv_std: float
    seed: int


def pad_rows(seqs: list[np.ndarray], pad_id: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Left-aligned padded batch of the given token rows."""
    S = max(len(s) for s in seqs)
    ids = np.full((len(seqs), S), pad_id, np.int32)
    mask = np.zeros((len(seqs), S), np.uint8)
    for r, s in enumerate(seqs):
        ids[r, : len(s)] = s
        mask[r, : len(s)] = 1
    return ids, mask


def _tok(rng, n, vocab):
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def _cfg1(seed=1):
    rng = np.random.default_rng(seed)
    V = 1000
    seqs = []
    for p in range(2):
        prompt = _tok(rng, 48, V)
        resps = [_tok(rng, int(rng.integers(16, 65)), V) for _ in range(4)]
        if p == 0:
            r0, r3 = resps[0], resps[3]
            m = int(rng.integers(1, min(len(r0), len(r3))))  # U[1, min-1]
            r3[:m] = r0[:m]
            if r3[m] == r0[m]:
                r3[m] = (r0[m] + 1) % V
        seqs += [np.concatenate([prompt, r]) for r in resps]
    ids, mask = pad_rows(seqs)
    return Workload("tiny-fwd", "1", ids, mask, 512, 1, 1, 64, "fp32", False, 1.0, seed)


def _grpo(seed, n_prompts, n_samples, M, name, config):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(n_prompts):
        prompt = _tok(rng, int(rng.integers(256, 1025)), VOCAB_BIG)
        for _ in range(n_samples):
            seqs.append(np.concatenate([prompt, _tok(rng, int(rng.integers(128, 2049)), VOCAB_BIG)]))
    ids, mask = pad_rows(seqs)
    return Workload(name, config, ids, mask, M, 32, 8, 128, "bf16", True, 1.0 / math.sqrt(128), seed)


def _cfg3(seed=3):
    rng = np.random.default_rng(seed)
    system = _tok(rng, 2048, VOCAB_BIG)
    seqs = []
    for _ in range(4):
        # each group: (member sample indices, shared token parts so far)
        groups = [(list(range(8)), [system])]
        for _turn in range(4):
            nxt = []
            for members, parts in groups:
                if len(members) >= 2 and rng.random() < 0.5:
                    h = len(members) // 2
                    for half in (members[:h], members[h:]):
                        nxt.append((half, parts + [_tok(rng, int(rng.integers(256, 1025)), VOCAB_BIG)]))
                else:
                    nxt.append((members, parts + [_tok(rng, int(rng.integers(256, 1025)), VOCAB_BIG)]))
            groups = nxt
        for members, parts in groups:
            for _m in members:
                seqs.append(np.concatenate(parts + [_tok(rng, int(rng.integers(256, 8193)), VOCAB_BIG)]))
    ids, mask = pad_rows(seqs)
    return Workload("multiturn-agentic", "3", ids, mask, 32768, 32, 8, 128, "bf16", True,
                    1.0 / math.sqrt(128), seed)


def _cfg4a(seed=4):
    rng = np.random.default_rng(seed)
    prefix = _tok(rng, 16384, VOCAB_BIG)
    firsts = rng.choice(VOCAB_BIG, size=64, replace=False).astype(np.int32)
    seqs = []
    for f in firsts:
        leaf = _tok(rng, 256, VOCAB_BIG)
        leaf[0] = f
        seqs.append(np.concatenate([prefix, leaf]))
    ids, mask = pad_rows(seqs)
    return Workload("deep-shared-16k+64x256", "4a", ids, mask, 32768, 32, 8, 128, "bf16", True,
                    1.0 / math.sqrt(128), seed)


def _cfg4b(seed=41):
    rng = np.random.default_rng(seed)
    firsts = rng.choice(VOCAB_BIG, size=16, replace=False).astype(np.int32)
    seqs = []
    for f in firsts:
        s = _tok(rng, 2048, VOCAB_BIG)
        s[0] = f
        seqs.append(s)
    ids, mask = pad_rows(seqs)
    return Workload("no-sharing-16x2048", "4b", ids, mask, 32768, 32, 8, 128, "bf16", True,
                    1.0 / math.sqrt(128), seed)


def make_workload(config: str) -> Workload:
    """Token batch of one named configuration ("1", "2", "3", "4a", "4b")."""
    config = str(config)
    if config == "1":
        return _cfg1()
    if config == "2":
        return _grpo(2, 16, 8, 8192, "grpo-16x8", "2")
    if config == "3":
        return _cfg3()
    if config == "4a":
        return _cfg4a()
    if config == "4b":
        return _cfg4b()
    raise ValueError(f"unknown config {config!r}")


def sweep_workload(L: int, b: int) -> Workload:
    """Config-5 point: GRPO generator, b samples per prompt, budget M = L."""
    n_prompts = math.ceil(4 * L / (640 + 1088 * b))
    seed = 5_000_000 + L * 10 + b
    w = _grpo(seed, n_prompts, b, L, f"sweep-L{L}-b{b}", "5")
    return w


def worked_example():
    """The pages' packing figure: Seq0 [A,B,C,D], Seq1 [A,B,E,F],
    Seq2 [A,G,H], with A..H encoded as ids 1..8 (0 is the pad id)."""
    A, B, C, D, E, F, G, H = range(1, 9)
    return pad_rows([np.array(s, np.int32) for s in ([A, B, C, D], [A, B, E, F], [A, G, H])])


def attention_inputs(L: int, hq: int, hkv: int, d: int, dtype: str, std: float, seed: int,
                     backward: bool = True):
    """Q, K, V (and dO) for one packed trie of length L, drawn in fp32 from a
    seeded ``torch.Generator`` on the CPU and rounded to the kernel dtype:
    Q [L,hq,d], K/V [L,hkv,d] ~ N(0,1)*std, dO [L,hq,d] ~ N(0,1).
    Returns CPU torch tensors of dtype bf16 or fp32."""
    import torch

    g = torch.Generator().manual_seed(int(seed))
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    q = (torch.randn(L, hq, d, generator=g) * std).to(tdt)
    k = (torch.randn(L, hkv, d, generator=g) * std).to(tdt)
    v = (torch.randn(L, hkv, d, generator=g) * std).to(tdt)
    do = torch.randn(L, hq, d, generator=g).to(tdt) if backward else None
    return q, k, v, do


SMALL_KINDS = ("grpo-small", "deep-small", "nested", "disjoint-small", "multiturn-small")


def small_workload(kind: str, seed: int = 0):
    """Scaled-down batches (a few hundred to a few thousand tokens) whose
    node boundaries fall inside 128-token tiles, for elementwise parity.
    Returns (ids, mask, max_tokens_per_mb)."""
    rng = np.random.default_rng(10_000 + 97 * SMALL_KINDS.index(kind) + seed)
    V = 50_000
    seqs = []
    if kind == "grpo-small":
        for _ in range(4):
            p = _tok(rng, int(rng.integers(64, 301)), V)
            seqs += [np.concatenate([p, _tok(rng, int(rng.integers(20, 401)), V)]) for _ in range(4)]
        M = 2048
    elif kind == "deep-small":
        prefix = _tok(rng, 300, V)
        leaves = [_tok(rng, int(rng.integers(50, 201)), V) for _ in range(6)]
        leaves.append(np.concatenate([leaves[0][:30], _tok(rng, 70, V)]))  # a branch inside a leaf
        seqs = [np.concatenate([prefix, lf]) for lf in leaves]
        M = 2048
    elif kind == "nested":
        base = _tok(rng, 90, V)
        seqs = [base[:40], base[:90], np.concatenate([base, _tok(rng, 150, V)]), base[:41],
                np.concatenate([base[:60], _tok(rng, 200, V)]), base[:90]]  # includes a duplicate
        M = 1024
    elif kind == "disjoint-small":
        seqs = [_tok(rng, int(n), V) for n in (37, 300, 129, 1, 255, 200)]
        for i, s in enumerate(seqs):
            s[0] = V + i  # distinct first tokens
        M = 1280
    elif kind == "multiturn-small":
        system = _tok(rng, 160, V)
        groups = [(list(range(4)), [system]) for _ in range(2)]
        for _turn in range(3):
            nxt = []
            for members, parts in groups:
                if len(members) >= 2 and rng.random() < 0.5:
                    h = len(members) // 2
                    for half in (members[:h], members[h:]):
                        nxt.append((half, parts + [_tok(rng, int(rng.integers(20, 81)), V)]))
                else:
                    nxt.append((members, parts + [_tok(rng, int(rng.integers(20, 81)), V)]))
            groups = nxt
        for members, parts in groups:
            for _m in members:
                seqs.append(np.concatenate(parts + [_tok(rng, int(rng.integers(20, 301)), V)]))
        M = 4096
    else:
        raise ValueError(kind)
    ids, mask = pad_rows(seqs)
    return ids, mask, M


def edge_layouts():
    """Degenerate batches: name -> (list of sequences, max_tokens_per_mb).

    one-token     a single one-token sequence (L = 128, 127 pads);
    three-copies  one 300-token sequence three times (one chain, three ids);
    full-trie     200 + 56 tokens filling L = 256 to the last slot;
    causal-1000   one 1000-token sequence (8 blocks, the last ragged)."""
    rng = np.random.default_rng(77)
    one = [np.array([5], np.int32)]
    seq = rng.integers(1, 1000, 300).astype(np.int32)
    copies = [seq, seq.copy(), seq.copy()]
    a = rng.integers(1, 1000, 100).astype(np.int32)
    full = [np.concatenate([a, rng.integers(1, 1000, 100)]).astype(np.int32),
            np.concatenate([a[:44], rng.integers(1000, 2000, 56)]).astype(np.int32)]  # 200 + 56 = 256
    long = [rng.integers(1, 1000, 1000).astype(np.int32)]
    return {"one-token": (one, 128), "three-copies": (copies, 384), "full-trie": (full, 256),
            "causal-1000": (long, 1024)}


def score_ramp_inputs(L: int, hq: int, hkv: int, d: int, dtype: str):
    """Inputs whose scores grow along the key axis: q = 30 u + noise and
    k_j = c_j u + noise with a fixed unit vector u and c_j rising linearly
    from 0 to 1.5 sqrt(d), noise N(0, 0.25); v and dO ~ N(0, 1).  With
    scale 1/sqrt(d) the scores reach about 45 at the end of a row, so an
    online softmax's running max keeps rising.  Drawn in float64 from
    torch.Generator(5150), rounded to ``dtype``; CPU tensors."""
    import torch

    g = torch.Generator().manual_seed(5150)
    u = torch.randn(d, generator=g, dtype=torch.float64)
    u /= u.norm()
    a, c_max = 30.0, 1.5 * math.sqrt(d)
    c = torch.linspace(0.0, c_max, L, dtype=torch.float64)
    q = a * u + 0.5 * torch.randn(L, hq, d, generator=g, dtype=torch.float64)
    k = c[:, None, None] * u + 0.5 * torch.randn(L, hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(L, hkv, d, generator=g, dtype=torch.float64)
    do = torch.randn(L, hq, d, generator=g, dtype=torch.float64)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    return tuple(x.to(tdt) for x in (q, k, v, do))


def batch_attention_inputs(lengths, hq: int, hkv: int, d: int, dtype: str, std: float, base_seed: int = 1_000_000):
    """Q, K, V, dO of a batch laid end to end (the concatenated layout of
    tree_pack_concat): trie t's rows are ``attention_inputs(L_t, ...)``
    drawn with seed base_seed + t.  CPU tensors."""
    import torch

    parts = [attention_inputs(Lt, hq, hkv, d, dtype, std, base_seed + t) for t, Lt in enumerate(lengths)]
    out = tuple(torch.cat([p[j] for p in parts]) for j in range(4))
    del parts
    return out


def device_attention_inputs(L: int, hq: int, hkv: int, d: int, std: float, seed: int, device):
    """bf16 Q, K, V ~ N(0, 1) * std and dO ~ N(0, 1), drawn on ``device``
    from a seeded device generator (for launches too large to draw on the
    host quickly).  Copy them to the host to give the oracle the same
    values."""
    import torch

    g = torch.Generator(device=device).manual_seed(int(seed))
    out = []
    for shape, s in (((L, hq, d), std), ((L, hkv, d), std), ((L, hkv, d), std), ((L, hq, d), 1.0)):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append((t * s).to(torch.bfloat16) if s != 1.0 else t.to(torch.bfloat16))
        del t
    return tuple(out)
