"""Dense numpy brute force used to pin the oracle.

It works on the generator's LOGICAL rows (DecodeCase.dense_kv: the rows in
token order, from the generator's own page placement), so it never touches a
page table or does any page arithmetic, and it uses numpy matrix products
and scipy's logsumexp/softmax instead of the oracle's loops."""
import numpy as np
from scipy.special import logsumexp, softmax

from workloads import bf16_bits_to_f32


def e4m3_codes_to_f64(codes):
    """OCP e4m3 codes -> values through PyTorch's float8_e4m3fn dtype (a
    library conversion, independent of the oracle's own decoding)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def dequant_rows(k, ks):
    if ks is None:
        return bf16_bits_to_f32(k).astype(np.float64)
    if k.dtype == np.uint8:   # e4m3 codes
        return e4m3_codes_to_f64(k) * ks.astype(np.float64)[..., None]
    return k.astype(np.float64) * ks.astype(np.float64)[..., None]


def dense_attention(case):
    B, Hq, D = case.q.shape
    G = case.group
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    qf = bf16_bits_to_f32(case.q).astype(np.float64)
    for b in range(B):
        k, v, ks, vs = case.dense_kv(b)
        K = dequant_rows(k, ks)   # [L, Hkv, D]
        V = dequant_rows(v, vs)
        L = K.shape[0]
        for h in range(Hq):
            if L == 0:
                lse[b, h] = -np.inf
                continue
            s = float(case.scale) * (K[:, h // G, :] @ qf[b, h])
            w = softmax(s)
            out[b, h] = w @ V[:, h // G, :]
            lse[b, h] = logsumexp(s)
    return out, lse


def dense_verify(case, q_rows, cu_seqlens_q):
    """Multi-token decode by dense causal attention: query token i of request
    b (row cu[b] + i) sees the first L_b - n_b + i + 1 logical rows."""
    T, Hq, D = q_rows.shape
    G = case.group
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    qf = bf16_bits_to_f32(q_rows).astype(np.float64)
    for b in range(case.batch):
        k, v, ks, vs = case.dense_kv(b)
        K = dequant_rows(k, ks)
        V = dequant_rows(v, vs)
        L = K.shape[0]
        r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n = r1 - r0
        for i in range(n):
            vis = min(max(L - n + i + 1, 0), L)
            if vis == 0:
                continue
            for h in range(Hq):
                s = float(case.scale) * (K[:vis, h // G, :] @ qf[r0 + i, h])
                out[r0 + i, h] = softmax(s) @ V[:vis, h // G, :]
                lse[r0 + i, h] = logsumexp(s)
    return out, lse
