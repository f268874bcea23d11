"""Error bound of decode over an 8-bit (E4M3) cache against the 16-bit oracle.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the benchmark's CPU-baseline leg use it.

Keeping historical K/V at reduced precision ("从零开始构建LLM推理引擎：模型执行器
深度解析", 5.2, KV缓存管理技巧) changes the attention result.  This module states
by how much, for the block quantiser the library implements (one fp32 scale
s = amax / 448 per (block, kv head), each value stored as the E4M3 code nearest
to x / s).

Ingredients.  E4M3 has 3 fraction bits and smallest normal exponent -6, so the
codes in the binade [2^e, 2^(e+1)) are 2^(e-3) apart and the nearest code to y
is within h(y) = 2^(max(e, -6) - 4) of it (e = floor(log2 |y|)); the stored
value x~ = s * code differs from x by at most s * h(x / s) (plus the fp32
rounding of the quotient, 2^-24 |x|).  Write dk[t][e], dv[t][d] for these
per-value errors of K and V, all within their half-steps hk, hv.

First order.  With scores z_t = scale * q . k_t, weights p_t = softmax(z)_t and
output o = sum_t p_t v_t, the score errors dz_t = scale * q . dk_t move the
weights to p~_t = p_t e^(dz_t) / sum_u p_u e^(dz_u), and since
sum_t p_t (v_t - o) = 0,
    o~_d - o_d = sum_t p_t dz_t (v_td - o_d) + sum_t p_t dv_td + (second order).
Both sums are linear in the independent rounding errors; treating each error
as a zero-mean variable bounded by its half-step (the usual model of rounding
random data), Hoeffding's inequality bounds the first-order part by c * S_d
with
    S_d^2 = sum_t p_t^2 [ (v_td - o_d)^2 s_t^2 + hv_td^2 ],
    s_t^2 = scale^2 sum_e q_e^2 hk_te^2,
except with probability 2 exp(-c^2 / 2) per output element (c = 7: 5e-11).

Second order.  The rest is sum_t p_t (e^(r_t) - 1 - r_t)(v_t - o) plus the
cross term (p~_t - p_t) dv_t, with r_t = dz_t - log sum_u p_u e^(dz_u); each
is quadratic in the score errors, whose typical size is s_t.  The allowance is
    Q_d = 4 max_t s_t^2 * sqrt(sum_t p_t (v_td - o_d)^2),
four times the size of its leading term (sum_t p_t (r_t^2 / 2)|v_td - o_d| with
r_t^2 ~ 2 s_t^2 and Cauchy-Schwarz on the weighted absolute deviation).  It is
an allowance for terms of that order, not a proof; the pins in the tests check
the whole bound against the exact difference of the 8-bit and 16-bit oracles.

The tolerance of an 8-bit GPU output against the 16-bit oracle is then
    |o8_gpu - o16| <= 2e-3 + c S_d + Q_d
(2e-3: the kernel against the oracle on the same codes, the bar of every decode
test).
"""
from __future__ import annotations

import math

import numpy as np

C_HOEFFDING = 7.0
Q_FACTOR = 4.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_FRACTION_BITS = 3


def e4m3_half_step(y):
    """Half the spacing of E4M3 codes in the binade of |y| (at least the subnormal step's half).

    A quotient within 2^-20 (relative) below a power of two is given the larger binade's
    half-step, so that fp32 rounding of y can never put it in a finer binade than assumed.
    Takes and returns numpy arrays, or float64 torch tensors.
    """
    import torch
    as_numpy = not isinstance(y, torch.Tensor)
    t = torch.as_tensor(np.asarray(y, dtype=np.float64)) if as_numpy else y.double()
    a = t.abs() * (1.0 + 2.0 ** -20)
    _, ex = torch.frexp(a)                    # a = m 2^ex, m in [0.5, 1): binade exponent ex - 1
    e = torch.clamp(ex - 1, min=E4M3_MIN_NORMAL_EXP)
    e = torch.where(a > 0, e, torch.full_like(e, E4M3_MIN_NORMAL_EXP))
    h = torch.ldexp(torch.ones_like(a), e - (E4M3_FRACTION_BITS + 1))
    return h.numpy() if as_numpy else h


def value_half_steps(x, s):
    """Largest |x~ - x| for values x quantised with scales s (broadcastable; numpy or torch)."""
    import torch
    if isinstance(x, torch.Tensor):
        s = torch.as_tensor(s, dtype=torch.float64)
        return e4m3_half_step(x / s) * s + x.abs() * 2.0 ** -24
    s = np.asarray(s, dtype=np.float64)
    return e4m3_half_step(x / s) * s + np.abs(x) * 2.0 ** -24


def _gather(pool, blk):
    """Blocks blk of a pool (numpy array, or a torch tensor of any float dtype) as a float64
    CPU tensor."""
    import torch
    if isinstance(pool, np.ndarray):
        return torch.from_numpy(np.asarray(pool[blk], dtype=np.float64))
    idx = torch.from_numpy(blk).to(pool.device)
    return pool.index_select(0, idx).cpu().double()


def decode_bound(q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens, scale, num_kv_heads,
                 out16, lse16, c: float = C_HOEFFDING, q_factor: float = Q_FACTOR) -> np.ndarray:
    """Per-element allowance c S_d + Q_d (without the 2e-3 kernel term), float64 [B][Hq][D].

    q [B][Hq][D] float64; k_pool / v_pool [NB][Hkv][bs][D]: the 16-bit values (a numpy
    array, or a torch tensor, widened block by block to float64, which is exact);
    k_scale / v_scale [NB][Hkv]: the quantiser's scales; out16 [B][Hq][D] and lse16
    [B][Hq] (natural log): the 16-bit oracle's output on the same q, K, V.  The sums run
    in float64 torch CPU operations (multithreaded).
    """
    import torch
    q = torch.as_tensor(np.asarray(q, dtype=np.float64))
    out16 = torch.as_tensor(np.asarray(out16, dtype=np.float64))
    lse16 = torch.as_tensor(np.asarray(lse16, dtype=np.float64))
    k_scale = np.asarray(k_scale, dtype=np.float64)
    v_scale = np.asarray(v_scale, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = num_kv_heads
    G = Hq // Hkv
    bs = k_pool.shape[2]
    sc = float(np.float32(scale))
    tol = torch.zeros((B, Hq, D), dtype=torch.float64)
    for s in range(B):
        n = int(context_lens[s])
        if n == 0:
            continue
        nb = -(-n // bs)
        blk = np.asarray(block_tables[s, :nb], dtype=np.int64)
        # [Hkv][n][D] in logical token order, and the per-token scales [Hkv][n]
        K = _gather(k_pool, blk).permute(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
        V = _gather(v_pool, blk).permute(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
        ks = torch.from_numpy(np.repeat(k_scale[blk].T, bs, axis=1)[:, :n].copy())
        vs = torch.from_numpy(np.repeat(v_scale[blk].T, bs, axis=1)[:, :n].copy())
        hk2 = value_half_steps(K, ks[:, :, None]) ** 2
        hv2 = value_half_steps(V, vs[:, :, None]) ** 2
        qg = q[s].reshape(Hkv, G, D)                               # [Hkv][G][D]
        z = sc * torch.bmm(K, qg.transpose(1, 2))                  # [Hkv][n][G]
        p = torch.exp(z - lse16[s].reshape(Hkv, 1, G))
        st2 = sc * sc * torch.bmm(hk2, (qg * qg).transpose(1, 2))  # [Hkv][n][G]
        o = out16[s].reshape(Hkv, G, D)
        V2 = V * V
        a = p * p * st2                                            # [Hkv][n][G]
        at = a.transpose(1, 2)
        # sum_t a_t (v_td - o_d)^2, expanded
        dev_k = torch.bmm(at, V2) - 2.0 * o * torch.bmm(at, V) + o * o * at.sum(2, keepdim=True)
        S2 = dev_k.clamp(min=0.0) + torch.bmm((p * p).transpose(1, 2), hv2)
        pt = p.transpose(1, 2)
        var = (torch.bmm(pt, V2) - 2.0 * o * torch.bmm(pt, V) + o * o * pt.sum(2, keepdim=True)).clamp(min=0.0)
        Q = q_factor * st2.amax(1)[:, :, None] * var.sqrt()
        tol[s] = (c * S2.sqrt() + Q).reshape(Hq, D)
    return tol.numpy()


def hoeffding_failure_probability(c: float = C_HOEFFDING) -> float:
    """Per-element probability that the first-order part exceeds c S_d under the model."""
    return 2.0 * math.exp(-c * c / 2.0)
