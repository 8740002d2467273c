"""Helpers shared by the GPU tests: uploads, ring runs, sampled comparisons."""
import os
import sys

import numpy as np

import ra_synth as rs

_CACHE = {}


def torch_mod():
    import torch
    return torch


def dev_tensor(arr, dtype):
    """Upload a device-representation array (uint16 bf16 bits or float32)."""
    torch = torch_mod()
    if dtype == rs.DT_BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def torch_dtype(dtype):
    torch = torch_mod()
    return torch.bfloat16 if dtype == rs.DT_BF16 else torch.float32


def inputs(w, with_do=False, q_hosts_only=False):
    key = (w.cfg, w.seed_offset, w.q_scale, w.block_len, w.n_hosts, w.heads_q, w.heads_kv,
           w.head_dim, w.dtype, with_do, q_hosts_only, w.host_begin, w.host_end)
    if key not in _CACHE:
        if len(_CACHE) > 2:
            _CACHE.clear()
        print(f"[inputs] drawing {w.name}", flush=True)
        _CACHE[key] = rs.make_inputs(w, with_do=with_do, q_hosts_only=q_hosts_only)
    return _CACHE[key]


def dims_of(w):
    import long_context_transformers_amd as ra
    return ra.Dims(w.batch, w.heads_q, w.heads_kv, w.head_dim, w.block_len, w.dtype, 0.0)


def cfg_of(w, flags=0, delay_us=0):
    import long_context_transformers_amd as ra
    return ra.RingCfg(dims_of(w), w.n_hosts, w.host_begin, w.host_end, w.layout, w.mask, flags,
                      delay_us)


def run_ring_fwd(w, inp, flags=0, delay_us=0, separate_comm=True, tensors=None):
    """Run ra_ring_fwd for workload w; returns (O, lse, stats) on the device."""
    torch = torch_mod()
    import long_context_transformers_amd as ra
    cfg = cfg_of(w, flags, delay_us)
    if tensors is None:
        q0 = w.host_begin - inp.q_host_base
        q = dev_tensor(inp.q_dev[q0:q0 + w.n_active], w.dtype)
        k = dev_tensor(inp.k_dev, w.dtype)
        v = dev_tensor(inp.v_dev, w.dtype)
    else:
        q, k, v = tensors
    O = torch.empty((w.n_active, w.batch, w.heads_q, w.block_len, w.head_dim),
                    dtype=torch_dtype(w.dtype), device="cuda")
    lse = torch.empty((w.n_active, w.batch, w.heads_q, w.block_len), dtype=torch.float32,
                      device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.current_stream()
    ms = torch.cuda.Stream() if separate_comm else cs
    stats = ra.ring_fwd(cfg, q, k, v, O, lse, ws, cs, ms)
    torch.cuda.synchronize()
    return O, lse, stats


def sampled(O, lse, w, rows):
    """Gather (host, batch, head, row) samples in cref.row_desc order."""
    torch = torch_mod()
    idx = torch.as_tensor(rows, device=O.device)
    Os = O.index_select(3, idx).float().cpu().numpy().reshape(-1, w.head_dim).astype(np.float64)
    Ls = lse.index_select(3, idx).cpu().numpy().reshape(-1).astype(np.float64)
    return Os, Ls


def oracle_rows(w, inp, rows):
    from oracle import cref
    desc = cref.row_desc(range(w.host_begin, w.host_end), range(w.batch), range(w.heads_q), rows)
    O, lse, mx, l = cref.attn_rows(inp.q_f32, inp.k_f32, inp.v_f32, n_hosts=w.n_hosts,
                                   layout=w.layout, causal=w.mask, rows=desc,
                                   q_host_base=inp.q_host_base)
    return O, lse


# Every parity check's worst error against its tolerance, collected for the
# end-of-run summary (tests/conftest.py prints it, so margins are on record
# even though pytest captures the per-test output).
MARGINS = []


def report(name, tol=None, **vals):
    """Print a parity result.  With a tolerance (one value for every max_*
    entry, or a dict of entry -> tolerance) the entry with the largest
    error/tolerance ratio is recorded in MARGINS."""
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                         for k, v in vals.items()), flush=True)
    if tol is None:
        return
    tols = tol if isinstance(tol, dict) else {k: tol for k in vals if k.startswith("max")}
    worst = None
    for k, t in tols.items():
        e = float(vals[k])
        if worst is None or e / t > worst[0] / worst[1]:
            worst = (e, float(t), k)
    if worst is not None:
        MARGINS.append({"name": f"{name} [{worst[2]}]", "err": worst[0], "tol": worst[1]})
