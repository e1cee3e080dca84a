"""Chunked prefill and decode of one step run concurrently on two streams
(the decode launched first on a second stream, the prefill on the launch
stream, joined by events) give bit for bit the results of the same calls on
one stream: the kernels share no writable memory and their results do not
depend on scheduling.  Both are also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import TOL, decode_state, max_err, prefill_state, prefill_workspace, say

pytestmark = pytest.mark.gpu


def test_decode_first_two_streams_equal_one_stream():
    pre = synth.custom_prefill(340, prior=[1500, 40, 900], chunk=[128, 64, 100], Hq=64, Hkv=8,
                               D=128, block_size=16)
    dec = synth.cfg2(B=12)
    C = int(pre.chunk.max())
    pc, pq, qs, ptab, plens, pmx = prefill_state(pre)
    dc, dq, dtab, dlens, dmx = decode_state(dec)
    pws = prefill_workspace(len(pre.chunk), pre.shape.Hq, C, pc.desc)
    dws = torch.zeros(max(pkv.decode_workspace_bytes(dec.B, dec.shape.Hq, dmx, dc.desc), 1),
                      dtype=torch.uint8, device="cuda")
    say(f"[streams] prefill chunks {pre.chunk.tolist()} priors {pre.prior.tolist()}, "
        f"decode B={dec.B}")

    def run(two_streams):
        po = torch.empty(tuple(pq.shape), dtype=torch.float32, device="cuda")
        do = torch.empty((dec.B, dec.shape.Hq, dec.shape.D), dtype=torch.float32, device="cuda")
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        if two_streams:
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
        pkv.decode(dq, dc.k_cache, dc.v_cache, dtab, dlens, dec.shape.scale, do, dc.desc, dmx,
                   workspace=dws, stream=side if two_streams else None)
        pkv.prefill_chunk(pq, qs, pc.k_cache, pc.v_cache, ptab, plens, pre.shape.scale, po,
                          pc.desc, C, pmx, workspace=pws)
        if two_streams:
            ev2 = torch.cuda.Event()
            ev2.record(side)
            main.wait_event(ev2)
        torch.cuda.synchronize()
        return po, do

    p1, d1 = run(False)
    for r in range(3):
        p2, d2 = run(True)
        assert torch.equal(p1, p2) and torch.equal(d1, d2), r
    ref_p = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale)
    ref_d = oracle.decode(dec.q, dec.k, dec.v, dec.lens, dec.shape.scale)
    ep = float(np.max(np.abs(p1.cpu().numpy().astype(np.float64) - ref_p)))
    ed = max_err(d1, ref_d)
    say(f"  prefill err {ep:.3e}, decode err {ed:.3e}")
    assert ep <= TOL["bf16"] and ed <= TOL["bf16"]
