"""kvq_pv_matvec_noalloc (the value pass with its split partials in the library's own
device array, for callers that cannot allocate) against kvq_pv_matvec on the same cache
and logits, and both against the oracle: two calls in a row on one device, the second
with a smaller input, so partials left by the first call would show."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kvq_testlib import Case, assert_out_close

pytestmark = pytest.mark.gpu

D = 128


def _case(name):
    W = synth.WORKLOADS
    if name == "large":
        wl = W["llama3_8b_gqa_b16_64k"].with_(batch=3, n_q_heads=8, n_kv_heads=2, seq_len=9000)
        return Case(wl, seed=11, lens=[9000, 5000, 1], device="cuda")
    wl = W["llama7b_32k"].with_(n_q_heads=4, n_kv_heads=4, seq_len=700)
    return Case(wl, seed=12, lens=[700], device="cuda")


def test_noalloc_value_pass_matches_workspace_entry_point():
    import long_context_decode_kvq_amd as kvq
    for name in ("large", "small"):  # the second call is the smaller input
        case = _case(name)
        cache = case.build_gpu()
        bufs = kvq.DecodeBuffers(cache)
        kvq.qk_matvec(cache, case.q, bufs.logits)
        kvq.pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace)
        out_ws = bufs.out.clone()
        out_na = torch.full_like(bufs.out, float("nan"))
        kvq.pv_matvec_noalloc(cache, bufs.logits, out_na)
        torch.cuda.synchronize()
        n_terms = 2 * 1024 * (case.k + 2)
        got_ws, got_na = out_ws.cpu().numpy(), out_na.cpu().numpy()
        lg = bufs.logits.cpu().numpy()
        for b in range(case.wl.batch):
            n = int(case.lens[b])
            for hq in range(case.wl.n_q_heads):
                h = hq // case.wl.group
                c = case.oracle_stream(b, h)
                l64 = lg[b, hq, :n].astype(np.float64)
                vd = oracle.dequant_values(c.v_codes, c.v_idx, c.v_val, c.v_scale, case.cbv)
                ref = oracle.attend(l64, vd)
                scale = oracle.output_tolerance_scale(l64, c, case.cbv)
                assert_out_close(got_na[b, hq], ref, scale, what=f"noalloc {name} b={b} hq={hq}")
                # same kernels on the same inputs: equal up to the order of the outlier sums
                assert np.all(np.abs(got_na[b, hq] - got_ws[b, hq]) <= n_terms * 2.0 ** -24 * scale + 1e-30)
