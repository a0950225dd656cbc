"""Contiguous (un-paged) brute-force attention, used only to pin the paged oracle.

TEST INFRASTRUCTURE.  Written separately from ``paged_attention.py`` so that a
mistake in the paged oracle's gather, scaling or softmax cannot cancel here.

It follows the dense form on the pages: the KVCacheAttention listing of [P1]
("LLM推理优化实战：从KV Cache到Speculative Decoding，把延迟打下来", section
"KV Cache：推理加速的第一板斧") keeps the cache contiguous as
[batch, seq, heads, d_head] and takes softmax(q K^T * d_head^-0.5) V, which is the
equation of [P4] ("大模型推理加速与显存黑科技", §2).  KV heads are repeated to
the query heads in contiguous groups (the GQA reading; [P2] "主流优化策略").
"""
from __future__ import annotations

import numpy as np
from scipy.special import softmax


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """q [H_q][d], K and V [L][H_kv][d] (float64) -> out [H_q][d] (float64)."""
    Hq = q.shape[0]
    L, Hkv, d = K.shape
    if L == 0:
        return np.zeros((Hq, d))
    group = Hq // Hkv
    Kh = np.repeat(K.transpose(1, 0, 2), group, axis=0)   # [H_q][L][d]
    Vh = np.repeat(V.transpose(1, 0, 2), group, axis=0)
    logits = np.einsum("hd,hld->hl", q, Kh) * scale         # [H_q][L]
    probs = softmax(logits, axis=-1)
    return np.einsum("hl,hld->hd", probs, Vh)
