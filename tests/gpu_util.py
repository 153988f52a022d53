"""Helpers shared by the GPU tests: move a seeded case to the device, run the HIP path,
compare against the oracle with the stated tolerance."""
from __future__ import annotations

import sys

import numpy as np

import oracle

# Tolerance of the decode (bf16 inputs, fp32 accumulation):
#   out: |gpu - ref| <= ATOL + RTOL * |ref| elementwise;  lse: |gpu - ref| <= LSE_TOL
#   relative L2 error of out (diagnostic gate, stricter in practice): <= REL_L2
ATOL, RTOL, LSE_TOL, REL_L2 = 2e-2, 1e-2, 1e-3, 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(case, dev="cuda"):
    import torch
    if case.dtype == "bf16":
        q = torch.from_numpy(case.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        kv = torch.from_numpy(case.kv_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        q = torch.from_numpy(case.q).to(dev)
        kv = torch.from_numpy(case.kv).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(case.cache_seqlens).to(dev)
    return q, kv, bt, lens


def run(case, tensors=None, split=True, options=None, num_cus=0, decoder=None, sinks=None, indices=None):
    """Decode `case` through the C ABI; returns (out float64 [rows, 512], lse float64 [rows], decoder)."""
    import torch
    import mla_decode_03_amd as mla
    q, kv, bt, lens = tensors if tensors is not None else to_device(case)
    topk = 0 if indices is None else int(indices.shape[2])
    if decoder is None:
        decoder = mla.Decoder(q, kv, bt, causal=case.causal, split=split, options=options,
                              num_cus=num_cus, topk=topk)
    sk = None if sinks is None else torch.from_numpy(np.ascontiguousarray(sinks, np.float32)).to(q.device)
    ix = None if indices is None else torch.from_numpy(np.ascontiguousarray(indices, np.int32)).to(q.device)
    out, lse = decoder(q, kv, bt, lens, case.scale, sinks=sk, indices=ix)
    torch.cuda.synchronize()
    R = case.q_len * case.num_heads
    o = out.float().cpu().numpy().astype(np.float64).reshape(case.batch * R, 512)
    l = lse.cpu().numpy().astype(np.float64).reshape(case.batch * R)
    return o, l, decoder


def compare(o, l, ref_o, ref_l, what=""):
    """Assert the tolerance; returns the error summary."""
    assert o.shape == ref_o.shape and l.shape == ref_l.shape, (o.shape, ref_o.shape)
    fin = np.isfinite(ref_l)
    # rows with no visible key: out 0, lse -inf on both sides
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), what + ": empty-row pattern differs"
    assert np.all(o[~fin] == 0.0), what + ": empty rows must be zero"
    d = np.abs(o - ref_o)
    bound = ATOL + RTOL * np.abs(ref_o)
    bad = ~(d <= bound)
    max_abs = float(d.max()) if d.size else 0.0
    dl = np.abs(l[fin] - ref_l[fin])
    max_lse = float(dl.max()) if dl.size else 0.0
    den = float(np.linalg.norm(ref_o))
    rel_l2 = float(np.linalg.norm(o - ref_o) / den) if den > 0 else 0.0
    summary = dict(max_abs=max_abs, max_lse=max_lse, rel_l2=rel_l2, n=int(o.size))
    say("  %s: max|d|=%.3e max|dlse|=%.3e relL2=%.3e" % (what, max_abs, max_lse, rel_l2))
    assert not bad.any(), "%s: %d elements outside tolerance (max %.3e)" % (what, int(bad.sum()), max_abs)
    assert max_lse <= LSE_TOL, "%s: lse error %.3e" % (what, max_lse)
    assert rel_l2 <= REL_L2, "%s: relative L2 %.3e" % (what, rel_l2)
    return summary


def oracle_rows(case, rows=None, sinks=None, indices=None):
    """Oracle rows; `sinks` float32 [H] is widened exactly to float64."""
    sk = None if sinks is None else np.asarray(sinks, np.float32).astype(np.float64)
    return oracle.decode_case(case, rows=rows, sinks=sk, indices=indices)
