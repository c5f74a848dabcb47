"""Test helpers: marshal torch tensors into the oracle's storage arrays."""
import numpy as np
import torch


def raw(t):
    """torch tensor -> numpy array in oracle storage form (float32 values,
    uint16 bf16 patterns or uint8 e4m3 codes).  None passes through."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def oracle_inputs(inp):
    return {k: raw(v) for k, v in inp.items()}


def oracle_forward(O, cfg, inp, **kw):
    a = oracle_inputs(inp) if not isinstance(next(iter(inp.values())), np.ndarray) else inp
    return O.layer_forward(a["x"], a["W_r"], a["W1"], a["b1"], a["W2"], a["b2"], K=cfg.K,
                           act=cfg.act, w=cfg.w, router_bias=a.get("router_bias"),
                           select_bias=a.get("select_bias"), n_groups=cfg.n_groups,
                           topk_groups=cfg.topk_groups, renormalize=cfg.renormalize,
                           w1_scale=a.get("w1_scale"), w2_scale=a.get("w2_scale"), **kw)
