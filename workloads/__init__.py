"""Seeded synthetic inputs shaped like the workloads the pages describe.

This module draws random numbers and prepares inputs; it holds none of the
method's arithmetic (no codec, no recurrence, no rotation).  Both the GPU path
(tests, benchmark) and the CPU oracle take their inputs from here, and from
nowhere else.

Conventions:
  * numpy Generator(PCG64(seed)), one generator per workload, drawing in the
    order written in each function;
  * "L2-normalised" = g / ||g||_2 over the last axis, in fp32;
  * bf16 inputs are rounded to nearest-even in numpy, so both sides see the
    same bits: the returned fp32 array holds exactly the bf16 values and
    ``bf16_bits`` gives the 16-bit patterns for the device.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32


def bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(F32)


def bf16_round(x):
    """fp32 values rounded to the nearest bf16 value (returned as fp32)."""
    return bf16_to_f32(bf16_bits(x))


def l2norm(x):
    x = np.asarray(x, F32)
    return (x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=F32))).astype(F32)


def softplus(x):
    x = np.asarray(x, F32)
    return np.log1p(np.exp(x)).astype(F32)


def sigmoid(x):
    x = np.asarray(x, F32)
    return (F32(1) / (F32(1) + np.exp(-x))).astype(F32)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# Single head, fp32, decode loop from a zero state
# --------------------------------------------------------------------------
def single_head_fp32(T=256, d=64, seed=0):
    """q, k ~ N(0,1) then L2-normalised; v ~ N(0,1); alpha ~ U(0.90, 0.999);
    beta ~ U(0, 1); all fp32, shapes [T, d] / [T].  Zero initial state."""
    g = _rng(seed)
    q = l2norm(g.standard_normal((T, d), dtype=F32))
    k = l2norm(g.standard_normal((T, d), dtype=F32))
    v = g.standard_normal((T, d), dtype=F32)
    alpha = g.uniform(0.90, 0.999, T).astype(F32)
    beta = g.uniform(0.0, 1.0, T).astype(F32)
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}


# --------------------------------------------------------------------------
# Decode batch: int8 state + partially filled window buffers
# --------------------------------------------------------------------------
def decode_batch(B=64, H=32, dk=128, dv=128, W=64, seed=0, fill=None, poison=True):
    """One decode step's inputs.

    Draw order: state [B,H,dv,dk] ~ N(0, sigma=0.5) (fp32; the caller
    quantises it); fill [B] ~ integer U{0..W-1}; buffer k [B,H,W,dk] ~ N(0,1)
    L2-normalised, v [B,H,W,dv] ~ N(0,1), alpha [B,H,W] ~ U(0.9,0.999),
    beta [B,H,W] ~ U(0,1) (all fp32; slots >= fill set to NaN when
    `poison`); q, k [B,H,dk] ~ N(0,1) L2-normalised, v [B,H,dv] ~ N(0,1),
    rounded to bf16; alpha, beta [B,H] as above.
    `fill` may be given (an int or an array) to override the drawn fill.
    """
    g = _rng(seed)
    state = (g.standard_normal((B, H, dv, dk), dtype=F32) * F32(0.5)).astype(F32)
    drawn_fill = g.integers(0, W, B).astype(np.int32)
    if fill is None:
        fill = drawn_fill
    else:
        fill = np.broadcast_to(np.asarray(fill, np.int32), (B,)).copy()
    bk = l2norm(g.standard_normal((B, H, W, dk), dtype=F32))
    bv = g.standard_normal((B, H, W, dv), dtype=F32)
    ba = g.uniform(0.9, 0.999, (B, H, W)).astype(F32)
    bb = g.uniform(0.0, 1.0, (B, H, W)).astype(F32)
    if poison:
        dead = np.arange(W)[None, None, :] >= fill[:, None, None]  # [B, 1, W]
        bk = np.where(dead[..., None], F32(np.nan), bk).astype(F32)
        bv = np.where(dead[..., None], F32(np.nan), bv).astype(F32)
        ba = np.where(dead, F32(np.nan), ba).astype(F32)
        bb = np.where(dead, F32(np.nan), bb).astype(F32)
    q = bf16_round(l2norm(g.standard_normal((B, H, dk), dtype=F32)))
    k = bf16_round(l2norm(g.standard_normal((B, H, dk), dtype=F32)))
    v = bf16_round(g.standard_normal((B, H, dv), dtype=F32))
    alpha = g.uniform(0.9, 0.999, (B, H)).astype(F32)
    beta = g.uniform(0.0, 1.0, (B, H)).astype(F32)
    return {"state": state, "fill": fill, "buf_k": bk, "buf_v": bv, "buf_alpha": ba,
            "buf_beta": bb, "q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}


def decode_tokens(B=64, H=32, dk=128, dv=128, step=0, seed=0):
    """Per-step decode inputs for a long decode run, from default_rng([seed, step]):
    q, k [B,H,dk] ~ N(0,1) L2-normalised, v [B,H,dv] ~ N(0,1) (bf16-rounded),
    alpha ~ U(0.9,0.999), beta ~ U(0,1) [B,H] fp32."""
    g = np.random.default_rng([seed, step])
    q = bf16_round(l2norm(g.standard_normal((B, H, dk), dtype=F32)))
    k = bf16_round(l2norm(g.standard_normal((B, H, dk), dtype=F32)))
    v = bf16_round(g.standard_normal((B, H, dv), dtype=F32))
    alpha = g.uniform(0.9, 0.999, (B, H)).astype(F32)
    beta = g.uniform(0.0, 1.0, (B, H)).astype(F32)
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}


# --------------------------------------------------------------------------
# Chunked prefill inputs
# --------------------------------------------------------------------------
def gdn_prefill(B=4, T=8192, H=16, dk=128, dv=128, seed=0):
    """q, k ~ N(0,1) L2-normalised, v ~ N(0,1), all rounded to bf16
    ([B,T,H,d]); x = 0.5*N(0,1) - 3, alpha = exp(-softplus(x));
    beta = sigmoid(N(0,1)); alpha, beta fp32 [B,T,H].  Zero initial state."""
    g = _rng(seed)
    q = bf16_round(l2norm(g.standard_normal((B, T, H, dk), dtype=F32)))
    k = bf16_round(l2norm(g.standard_normal((B, T, H, dk), dtype=F32)))
    v = bf16_round(g.standard_normal((B, T, H, dv), dtype=F32))
    x = (F32(0.5) * g.standard_normal((B, T, H), dtype=F32) - F32(3.0)).astype(F32)
    alpha = np.exp(-softplus(x)).astype(F32)
    beta = sigmoid(g.standard_normal((B, T, H), dtype=F32))
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}


def gdn_prefill_varlen(lengths, H=16, dk=128, dv=128, seed=0):
    """A packed batch of sequences of the given lengths: the gdn_prefill
    distributions over sum(lengths) tokens laid back to back ([T,H,d],
    alpha and beta [T,H]) and cu_seqlens (int32, B+1 offsets)."""
    lengths = [int(n) for n in lengths]
    x = gdn_prefill(B=1, T=sum(lengths), H=H, dk=dk, dv=dv, seed=seed)
    out = {key: val[0] for key, val in x.items()}
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return out


def ssd_prefill(B=2, T=4096, H=80, dk=128, dv=64, seed=0, outlier_channels=0,
                outlier_gain=20.0):
    """q, k ~ N(0,1) [B,T,H,dk] and v ~ N(0,1) [B,T,H,dv], rounded to bf16
    (not normalised); a = exp(-softplus(-3 + 0.5*N(0,1))) fp32 [B,T,H].
    `outlier_channels` > 0 multiplies that many leading channels of q and k
    by `outlier_gain` before rounding (accuracy probe only)."""
    g = _rng(seed)
    q = g.standard_normal((B, T, H, dk), dtype=F32)
    k = g.standard_normal((B, T, H, dk), dtype=F32)
    v = g.standard_normal((B, T, H, dv), dtype=F32)
    if outlier_channels:
        q[..., :outlier_channels] *= F32(outlier_gain)
        k[..., :outlier_channels] *= F32(outlier_gain)
    x = (F32(-3.0) + F32(0.5) * g.standard_normal((B, T, H), dtype=F32)).astype(F32)
    a = np.exp(-softplus(x)).astype(F32)
    return {"q": bf16_round(q), "k": bf16_round(k), "v": bf16_round(v), "alpha": a}
