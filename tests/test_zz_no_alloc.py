"""mla_decode_noalloc (plan and split partials in the library's static device scratch)
against mla_get_metadata + mla_decode_ex with a caller-owned plan and workspace: bit for
bit, on two calls in a row (the second smaller, so the scratch still holds the first
call's plan and partials), and both against the oracle."""
import ctypes

import numpy as np
import pytest

from gpu_util import compare, oracle_rows, run, say, to_device
from mla_inputs import make_case, make_sinks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_03_amd as mla
    mla.lib()


def _noalloc(case, tensors, sinks=None):
    import torch
    import mla_decode_03_amd as mla
    q, kv, bt, lens = tensors
    prob = mla.make_problem(q, kv, bt, causal=case.causal)
    B, T, H = case.batch, case.q_len, case.num_heads
    out = torch.full((B, T, H, 512), float("nan"), dtype=q.dtype, device=q.device)
    lse = torch.full((B, T, H), float("nan"), dtype=torch.float32, device=q.device)
    sk = None if sinks is None else torch.from_numpy(np.ascontiguousarray(sinks, np.float32)).to(q.device)
    mla.decode_noalloc(prob, q, kv, bt, lens, case.scale, out, lse, sinks=sk)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64).reshape(B * T * H, 512)
    l = lse.cpu().numpy().astype(np.float64).reshape(B * T * H)
    return o, l


CASES = [
    # (B, T, H, lens, causal, dtype, sinks): the second of each pair is the smaller input
    [(64, 1, 128, None, False, "bf16", False), (3, 2, 16, [130, 2, 65], True, "bf16", False)],
    [(9, 1, 128, [3000, 1, 64, 4097, 0, 700, 8000, 129, 2000], False, "bf16", True),
     (2, 1, 48, [77, 300], False, "bf16", True)],
    [(2, 2, 16, [300, 65], True, "f32", False), (1, 1, 16, [40], False, "f32", False)],
]


@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_matches_the_planned_decode(pair):
    for i, (B, T, H, lens, causal, dtype, with_sinks) in enumerate(CASES[pair]):
        if lens is None:
            rng = np.random.default_rng(5)
            lens = [int(x) for x in rng.integers(1, 4097, size=B)]
        case = make_case(batch=B, q_len=T, num_heads=H, seqlens=lens, dtype=dtype, causal=causal,
                         seed=900 + 10 * pair + i)
        sinks = make_sinks(H, seed=pair + i) if with_sinks else None
        say("noalloc", pair, i, B, T, H, dtype, "sinks" if with_sinks else "")
        t = to_device(case)
        o_ref, l_ref, _ = run(case, tensors=t, sinks=sinks)      # caller-owned plan and workspace
        o, l = _noalloc(case, t, sinks)
        assert np.array_equal(o, o_ref, equal_nan=True), "out differs from the planned decode"
        assert np.array_equal(l, l_ref, equal_nan=True), "lse differs from the planned decode"
        ref_o, ref_l = oracle_rows(case, sinks=sinks)
        compare(o, l, ref_o, ref_l, "noalloc %d/%d" % (pair, i))


def test_noalloc_refuses_what_does_not_fit():
    """A batch whose plan metadata exceeds the scratch, and a sparse problem, are refused
    before anything is enqueued."""
    import torch
    import mla_decode_03_amd as mla
    from mla_decode_03_amd import _abi
    L = mla.lib()
    big = mla.Problem(batch=70000, q_len=1, num_heads=16, causal=0, num_pages=1, block_table_stride=1,
                      max_blocks_per_seq=1, dtype=mla.DTYPE_BF16)
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(x.data_ptr())
    rc = L.mla_decode_noalloc(ctypes.byref(big), None, p, p, p, p, ctypes.c_float(1.0), p, p, None)
    assert rc == _abi.MLA_ERR_WORKSPACE
    sp = mla.Problem(batch=2, q_len=1, num_heads=16, causal=0, num_pages=4, block_table_stride=2,
                     max_blocks_per_seq=2, dtype=mla.DTYPE_BF16, topk=64)
    rc = L.mla_decode_noalloc(ctypes.byref(sp), None, p, p, p, p, ctypes.c_float(1.0), p, p, None)
    assert rc == _abi.MLA_ERR_UNSUPPORTED
