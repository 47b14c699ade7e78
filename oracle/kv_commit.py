"""Oracle: committing a verified block to the shared KV cache.  Test
infrastructure only.

Source: Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法" (the
AR path verifies the proposed block and keeps the longest valid prefix; the
first token of a block is generated with the AR weights alone) and section
"实验" (drafting and verification share one KV cache).

Readings taken here (the pages do not spell the cache update out):
* the rows a step may keep are its clean rows: they carry the adapter gate 0
  and see only the cache and earlier clean rows, so their keys and values are
  exactly those of the AR model at those positions;
* after verification with L accepted drafts, sequence b keeps clean rows
  0..L (the block's AR token and the accepted drafts), appended after its
  cache_len[b] valid rows; the noisy rows and the rejected clean rows are
  dropped;
* the correction (or bonus) token is not written: it is the next block's
  first clean row;
* a cache with C rows of capacity keeps the block's rows only if all of them
  fit (cache_len[b] + L + 1 <= C); a sequence whose kept rows do not fit, or
  that is already flagged (L = -1), keeps nothing and is flagged
  (accept_len -1): dropping emitted tokens from the cache silently would
  leave it out of step with the text.

Float64 arrays (any dtype the caller passes is kept).
"""

import numpy as np


def kv_commit(k_cache, v_cache, cache_len, k_clean, v_clean, accept_len):
    """k_cache/v_cache [B, C, Hkv, D]; cache_len [B]; k_clean/v_clean
    [B, block, Hkv, D] (the step's clean rows); accept_len [B] in -1..block-1.

    Returns (k_cache', v_cache', cache_len', accept_len') as new arrays: rows
    cache_len[b] + j of sequence b take clean row j for j <= accept_len[b]
    and cache_len'[b] = cache_len[b] + accept_len[b] + 1, when those rows fit
    the capacity C; otherwise sequence b is unchanged and accept_len'[b] = -1."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    cap = kc.shape[1]
    lens = np.array(cache_len, dtype=np.int64, copy=True)
    acc = np.array(accept_len, dtype=np.int64, copy=True)
    for b in range(kc.shape[0]):
        keep = int(acc[b]) + 1
        if keep <= 0 or int(cache_len[b]) + keep > cap:
            acc[b] = -1
            continue
        for j in range(keep):
            slot = int(cache_len[b]) + j
            kc[b, slot] = k_clean[b, j]
            vc[b, slot] = v_clean[b, j]
        lens[b] = int(cache_len[b]) + keep
    return kc, vc, lens, acc
