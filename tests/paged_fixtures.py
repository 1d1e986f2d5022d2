"""Tiny paged caches built by hand from contiguous per-sequence K/V, for the oracle pins.

The placement loop here is test code: it puts logical token t of a sequence
at (table[t // 16], t % 16) of a pool whose physical ids come from a random
permutation, poisoning every other slot with NaN.
"""
import numpy as np

BS = 16


def place(seqs_k, seqs_v, num_blocks, rng, shared=None, dtype=np.float32):
    """seqs_k[s]: [L_s, Hkv, D] contiguous keys (same for values).

    shared: optional (n_tokens_shared) -- the first n tokens of every sequence
    are identical and stored once in shared blocks (n must be a multiple of 16).
    Returns (k_cache, v_cache, tables[B, maxb], lens).
    """
    hkv, d = seqs_k[0].shape[1], seqs_k[0].shape[2]
    kc = np.full((num_blocks, hkv, BS, d), np.nan, dtype=dtype)
    vc = np.full((num_blocks, hkv, BS, d), np.nan, dtype=dtype)
    perm = list(rng.permutation(num_blocks))
    lens = [k.shape[0] for k in seqs_k]
    maxb = max(1, max(-(-L // BS) for L in lens))
    tables = np.zeros((len(lens), maxb), dtype=np.int32)
    shared_ids = []
    if shared:
        assert shared % BS == 0
        shared_ids = [perm.pop() for _ in range(shared // BS)]
    for s, L in enumerate(lens):
        ids = []
        for j in range(-(-L // BS)):
            if j < len(shared_ids):
                ids.append(shared_ids[j])
            else:
                ids.append(perm.pop())
        tables[s, :len(ids)] = ids
        for t in range(L):
            b, o = ids[t // BS], t % BS
            kc[b, :, o, :] = seqs_k[s][t]
            vc[b, :, o, :] = seqs_v[s][t]
    # padding entries point at a still-unused block
    pad = perm[-1] if perm else 0
    for s, L in enumerate(lens):
        tables[s, -(-L // BS):] = pad
    return kc, vc, tables, np.array(lens, dtype=np.int32)


def relabel(kc, vc, tables, rng):
    """Move every physical block to a new id by a random permutation and rewrite the tables."""
    nb = kc.shape[0]
    pi = rng.permutation(nb)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    return kc2, vc2, pi[tables].astype(np.int32)
