"""Shared helpers for the parity tests: seeded inputs, tolerances, metrics."""

import dataclasses

import numpy as np

from workloads import Workload, draw_inputs

# Tolerances (the fp32 gate is relative to max|ref| on every output; bf16:
# O and LSE by max error relative to max|ref|, gradients by relative
# Frobenius error).
F32_MAX_REL = 1e-5
BF16_O_MAX_REL = 2e-2
BF16_LSE_MAX_REL = 2e-2
BF16_GRAD_FRO_REL = 3e-2


def make_case(B, H, n, d, dtype, window=-1, q_mult=1.0, seed=12345, kv_heads=0):
    kv = f"kv{kv_heads}" if kv_heads else ""
    return Workload(f"case_b{B}h{H}{kv}n{n}d{d}_{dtype}_w{window}", B, H, n, d, dtype, window=window,
                    q_mult=q_mult, seed=seed, kv_heads=kv_heads)


def to_device(arrs, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(v).to(device="cuda", dtype=tdt).contiguous() for k, v in arrs.items()}


def max_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def fro_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def check_outputs(dtype, got, ref, label=""):
    """got/ref: dicts with any of o, lse, dq, dk, dv.  Returns error dict;
    raises AssertionError naming the first output over its tolerance.

    A gradient whose exact value is identically zero (dQ and dK at window 0;
    the fp64 oracle then returns zeros or ~1e-16 rounding residue) has no
    relative error; it is measured against the largest gradient reference of
    the problem instead."""
    errs = {}
    grad_scale = max([float(np.max(np.abs(ref[k]))) for k in ("dq", "dk", "dv") if k in ref] + [0.0])
    for key in ("o", "lse", "dq", "dk", "dv"):
        if key not in got:
            continue
        if key in ("dq", "dk", "dv") and float(np.max(np.abs(ref[key]))) <= 1e-12 * grad_scale:
            e = float(np.max(np.abs(got[key]))) / max(grad_scale, 1e-30)
            tol = F32_MAX_REL if dtype == "f32" else BF16_GRAD_FRO_REL
        elif dtype == "f32":
            e, tol = max_rel(got[key], ref[key]), F32_MAX_REL
        elif key == "o":
            e, tol = max_rel(got[key], ref[key]), BF16_O_MAX_REL
        elif key == "lse":
            e, tol = max_rel(got[key], ref[key]), BF16_LSE_MAX_REL
        else:
            e, tol = fro_rel(got[key], ref[key]), BF16_GRAD_FRO_REL
        errs[key] = e
        assert np.all(np.isfinite(got[key])), f"{label} {key}: non-finite values"
        assert e <= tol, f"{label} {key}: error {e:.3e} > tolerance {tol:.1e}"
    return errs


def run_gpu(wl, inputs, backward=True):
    """Run the HIP path on the given float32 host inputs; returns numpy fp32."""
    import torch
    import exact_attention_69_amd as ea
    t = to_device(inputs, wl.dtype)
    gqa = wl.Hkv != wl.H
    fwd, bwd = (ea.attn_fwd_gqa, ea.attn_bwd_gqa) if gqa else (ea.attn_fwd, ea.attn_bwd)
    o, lse = fwd(t["q"], t["k"], t["v"], wl.scale, wl.window)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = bwd(t["q"], t["k"], t["v"], o, t["do"], lse, wl.scale, wl.window)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def oracle_case(wl, inputs, heads=None):
    """Full oracle on all heads (or on the listed flat head indices; with
    shared key/value heads, on the listed flat key/value heads together with
    all query heads of their groups)."""
    import oracle
    q, k, v, do = (inputs[x] for x in ("q", "k", "v", "do"))
    if wl.Hkv != wl.H:
        G = wl.group
        if heads is not None:
            qsel = lambda a: a.reshape(-1, G, wl.n, wl.d)[heads]
            ksel = lambda a: a.reshape(-1, 1, wl.n, wl.d)[heads]
            q, do, k, v = qsel(q), qsel(do), ksel(k), ksel(v)
        O, lse = oracle.attention_forward_gqa(q, k, v, wl.scale, wl.window)
        dq, dk, dv = oracle.attention_backward_gqa(q, k, v, do, wl.scale, wl.window)
        return {"o": O, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    if heads is not None:
        sel = lambda a: a.reshape(-1, wl.n, wl.d)[heads]
        q, k, v, do = sel(q), sel(k), sel(v), sel(do)
    O, lse = oracle.attention_forward(q, k, v, wl.scale, wl.window)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, wl.scale, wl.window)
    return {"o": O, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def select_heads(outs, wl, heads):
    """The outputs of the flat heads ``heads`` in the layout oracle_case
    returns for them (with shared key/value heads: key/value heads, each with
    its group of query heads)."""
    res = {}
    G = wl.group
    for key, a in outs.items():
        if key == "lse":
            res[key] = a.reshape(-1, G, wl.n)[heads] if G > 1 else a.reshape(-1, wl.n)[heads]
        elif key in ("dk", "dv") or G == 1:
            res[key] = a.reshape(-1, wl.n, wl.d)[heads]
            if G > 1:
                res[key] = res[key][:, None]
        else:
            res[key] = a.reshape(-1, G, wl.n, wl.d)[heads]
    return res


def invariant_errors(inputs, outs, wl):
    """Whole-tensor identities of the exact gradients, per key/value head, as
    ratios: sum_j dK_j = 0; sum_j dV_j = sum of dO over the rows of the
    group's query heads; sum over the group of <dQ,Q> = <dK,K>."""
    G = wl.group
    q = inputs["q"].reshape(-1, G * wl.n, wl.d).astype(np.float64)
    k = inputs["k"].reshape(-1, wl.n, wl.d).astype(np.float64)
    do = inputs["do"].reshape(-1, G * wl.n, wl.d).astype(np.float64)
    dq = outs["dq"].reshape(-1, G * wl.n, wl.d).astype(np.float64)
    dk = outs["dk"].reshape(-1, wl.n, wl.d).astype(np.float64)
    dv = outs["dv"].reshape(-1, wl.n, wl.d).astype(np.float64)
    sum_dk = np.linalg.norm(dk.sum(axis=1), axis=-1) / np.maximum(np.linalg.norm(dk, axis=-1).sum(axis=1), 1e-30)
    dv_err = np.linalg.norm(dv.sum(axis=1) - do.sum(axis=1), axis=-1) / np.maximum(
        np.linalg.norm(do, axis=-1).sum(axis=1), 1e-30)
    a = np.einsum("hid,hid->h", dq, q)
    b = np.einsum("hid,hid->h", dk, k)
    qk = np.abs(a - b) / np.maximum(np.abs(dq * q).sum(axis=(1, 2)) + np.abs(dk * k).sum(axis=(1, 2)), 1e-30)
    return {"sum_dk": float(sum_dk.max()), "sum_dv": float(dv_err.max()), "qdq_kdk": float(qk.max())}


__all__ = [n for n in dir() if not n.startswith("_")] + ["dataclasses", "draw_inputs"]
