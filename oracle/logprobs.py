"""Oracle: per-sequence log-probabilities and entropies gathered from the
logits of a trie-packed batch.  TEST INFRASTRUCTURE ONLY (see the package
docstring).

[TT] section "Log Probability 计算：树结构的特殊处理": labels cannot come
from rolling the packed input ids, because sequences share positions.  Each
sequence's own token order has to be recovered from the trie, and shared
prefixes should be computed once.  The pages' gather walks every sequence
of the trie and, for every node on its path, takes
  - internal log-probabilities: the logits at positions start .. end - 1 of
    the node predict the tokens at start + 1 .. end;
  - the transition log-probability: the logits at the parent node's last
    position predict the child node's first token;
both cached by their position keys, so sequences through a shared prefix
reuse them.  The pieces are concatenated in order into the sequence's own
vector, and the per-sequence results are merged back into the padded
(batch, length) layout, short sequences padded with a padding value.

Readings (the pages leave these open):
  - a sequence of l tokens has l - 1 predictions; row r of the merged
    output holds them in columns 0 .. l - 2 and the padding value after;
    the merged width is the input's S;
  - entropy is that of the full next-token distribution at the predicting
    position, -sum_v p_v log p_v, p = softmax(logits row), with 0 log 0 = 0;
  - everything is computed in float64 from the logits as given.
"""

from __future__ import annotations

import numpy as np

from .packing import PackedTrie


def _log_softmax(row: np.ndarray) -> np.ndarray:
    """Natural-log softmax of one logits row, max-shifted."""
    x = np.asarray(row, dtype=np.float64)
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def _entropy(row: np.ndarray) -> float:
    """-sum_v p_v log p_v, with 0 log 0 = 0 (a -inf logit contributes 0)."""
    ls = _log_softmax(row)
    p = np.exp(ls)
    with np.errstate(invalid="ignore"):  # 0 * -inf is computed, then discarded
        return float(-np.where(p > 0, p * ls, 0.0).sum())


def prediction_logprob_entropy(row: np.ndarray, label: int) -> tuple[float, float]:
    """One prediction: the log-probability of `label` under softmax(row) and
    the entropy of that distribution (the quantities every cached piece of
    the gather below holds)."""
    return float(_log_softmax(row)[label]), _entropy(row)


def gather_tree_logprobs_entropy(tries: list[PackedTrie], logits: list[np.ndarray], batch_size: int,
                                 max_len: int, padding_value: float = 0.0):
    """[TT] gather_packed_tree_logprobs_entropy and merge_packed_tree_results:
    `logits[t]` is the [L_t, V] logits of trie t (row p = the model's output
    at packed position p).  Returns (logp, entropy), each float64
    [batch_size, max_len], laid out as described in the module docstring."""
    logp = np.full((batch_size, max_len), padding_value, np.float64)
    ent = np.full((batch_size, max_len), padding_value, np.float64)
    for trie, lg in zip(tries, logits):
        internal: dict[tuple[int, int], tuple[list[float], list[float]]] = {}
        transition: dict[tuple[int, int], tuple[float, float]] = {}
        for k, row in enumerate(trie.seq_ids):
            a, b = int(trie.seq_iv_ptr[k]), int(trie.seq_iv_ptr[k + 1])
            lp_parts: list[float] = []
            en_parts: list[float] = []
            prev_end = None
            for start, end in trie.seq_iv[a:b]:
                start, end = int(start), int(end)
                if prev_end is not None:
                    # parent's last position predicts this node's first token
                    key = (prev_end, start)
                    if key not in transition:
                        transition[key] = prediction_logprob_entropy(lg[prev_end], trie.token_ids[start])
                    lp, en = transition[key]
                    lp_parts.append(lp)
                    en_parts.append(en)
                key = (start, end)
                if key not in internal:
                    preds = [prediction_logprob_entropy(lg[p], trie.token_ids[p + 1]) for p in range(start, end)]
                    internal[key] = ([a for a, _ in preds], [b for _, b in preds])
                lps, ens = internal[key]
                lp_parts.extend(lps)
                en_parts.extend(ens)
                prev_end = end
            n = len(lp_parts)
            logp[int(row), :n] = lp_parts
            ent[int(row), :n] = en_parts
    return logp, ent
