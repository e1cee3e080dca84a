"""The decode step and the chunked prefill captured in a HIP graph and
replayed: every replay must equal an eager call on the same inputs bit for
bit.  Between replays the inputs are changed by eager work and an eager call
runs, so a replay that read stale state or skipped a node would differ.  The
library records only kernel launches (no memsets or allocations)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from paged_kv_cache_indirected_amd.paged import to_device_rows
from harness import TOL, decode_state, max_err, prefill_state, prefill_workspace, say

pytestmark = pytest.mark.gpu


def _slots_of_last_rows(cache, lens, bs):
    return torch.tensor([cache.seqs.block_ids(b)[(int(L) - 1) // bs] * bs + (int(L) - 1) % bs
                         for b, L in enumerate(lens)], dtype=torch.int32, device="cuda")


def test_fused_decode_step_graph_replays_equal_eager():
    b = synth.cfg2(B=8)
    sh = b.shape
    say(f"[graph] fused append+decode, B={b.B}, lens={b.lens.tolist()}")
    cache, q, tables, lens, mx = decode_state(b)
    st = b.seq_start()
    last = st[1:] - 1
    k_new = to_device_rows(b.k[last], pkv.BF16, "cuda")
    v_new = to_device_rows(b.v[last], pkv.BF16, "cuda")
    slots = _slots_of_last_rows(cache, b.lens, sh.block_size)
    ws = torch.zeros(max(pkv.decode_workspace_bytes(b.B, sh.Hq, mx, cache.desc), 1),
                     dtype=torch.uint8, device="cuda")
    out_g = torch.empty((b.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)

    def call(out):
        pkv.append_decode(k_new, v_new, slots, q, cache.k_cache, cache.v_cache, tables, lens,
                          sh.scale, out, cache.desc, mx, workspace=ws)
    call(out_e)                       # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    gen = torch.Generator(device="cuda").manual_seed(5)
    for r in range(4):
        if r:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        call(out_e)
        torch.cuda.synchronize()
        say(f"  replay {r}: max |graph - eager| {(out_g - out_e).abs().max().item():.3e}")
        assert torch.equal(out_g, out_e)
    # The last replay's inputs against the oracle.
    ref = oracle.decode(q.view(torch.int16).cpu().numpy().view(np.uint16), b.k, b.v, b.lens,
                        sh.scale)
    assert max_err(out_g, ref) <= TOL["bf16"]


def test_key_split_prefill_graph_replays_equal_eager():
    # A short grid, so the library splits the keys: the prefill kernel and
    # the state merge are both captured.
    b = synth.custom_prefill(330, prior=[2000, 700], chunk=[48, 16], Hq=16, Hkv=2, D=128,
                             block_size=16)
    C = int(b.chunk.max())
    cache, q, qs, tables, lens, mx = prefill_state(b)
    ws = prefill_workspace(len(b.chunk), b.shape.Hq, C, cache.desc)
    assert ws is not None
    out_g = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)

    def call(out):
        pkv.prefill_chunk(q, qs, cache.k_cache, cache.v_cache, tables, lens, b.shape.scale, out,
                          cache.desc, C, mx, workspace=ws)
    call(out_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    gen = torch.Generator(device="cuda").manual_seed(6)
    for r in range(4):
        if r:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        call(out_e)
        torch.cuda.synchronize()
        say(f"  prefill replay {r}: max |graph - eager| "
            f"{(out_g - out_e).abs().max().item():.3e}")
        assert torch.equal(out_g, out_e)


def test_cascade_decode_graph_replays_equal_eager():
    # The cascade forks its prefix pass onto the library's side stream and
    # joins it back before the state merge: the capture must take in both
    # branches and the join.
    from test_gpu_cascade import _shared_batch
    B, P = 24, 16 * 40
    own = [(7 * i) % 90 for i in range(B)]
    sh, cache, qn, tab, lens, K, V, L, pids = _shared_batch(331, B, P, own, 16, 2, 128, 16)
    say(f"[graph] cascade decode, B={B}, prefix {P}")
    q = to_device_rows(qn, pkv.BF16, "cuda")
    nbp = P // sh.block_size
    tab_s = tab[:, nbp:].contiguous()
    lens_s = (lens - P).to(torch.int32).contiguous()
    mx = int(lens_s.max().item())
    pb = torch.tensor(pids[:nbp], dtype=torch.int32, device="cuda")
    ws = torch.empty(pkv.decode_cascade_workspace_bytes(B, sh.Hq, P, mx, cache.desc),
                     dtype=torch.uint8, device="cuda")
    out_g = torch.empty((B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)

    def call(out):
        pkv.decode_cascade(q, cache.k_cache, cache.v_cache, pb, P, tab_s, lens_s, sh.scale, out,
                           cache.desc, mx, workspace=ws)
    call(out_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for r in range(4):
        if r:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        call(out_e)
        torch.cuda.synchronize()
        say(f"  cascade replay {r}: max |graph - eager| "
            f"{(out_g - out_e).abs().max().item():.3e}")
        assert torch.equal(out_g, out_e)
    ref = oracle.decode(q.view(torch.int16).cpu().numpy().view(np.uint16), K, V, L, sh.scale)
    assert max_err(out_g, ref) <= TOL["bf16"]


def test_cascade_decode_on_a_side_stream_orders_later_work():
    # Called on a non-default stream and read back by work enqueued on that
    # stream only: the join must order the prefix pass before the merge and
    # the merge before the caller's next work.
    from test_gpu_cascade import _shared_batch
    B, P = 16, 16 * 24
    own = [(5 * i) % 70 for i in range(B)]
    sh, cache, qn, tab, lens, K, V, L, pids = _shared_batch(332, B, P, own, 16, 2, 128, 16)
    q = to_device_rows(qn, pkv.BF16, "cuda")
    nbp = P // sh.block_size
    tab_s = tab[:, nbp:].contiguous()
    lens_s = (lens - P).to(torch.int32).contiguous()
    mx = int(lens_s.max().item())
    pb = torch.tensor(pids[:nbp], dtype=torch.int32, device="cuda")
    ws = torch.empty(pkv.decode_cascade_workspace_bytes(B, sh.Hq, P, mx, cache.desc),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    copies = []
    with torch.cuda.stream(st):
        for _ in range(3):
            out.fill_(float("nan"))
            ws.fill_(0xFF)                # prefix states are NaN until the pass writes them
            pkv.decode_cascade(q, cache.k_cache, cache.v_cache, pb, P, tab_s, lens_s, sh.scale,
                               out, cache.desc, mx, workspace=ws)
            copies.append(out.clone())
    torch.cuda.synchronize()
    ref = oracle.decode(qn, K, V, L, sh.scale)
    for c in copies:
        assert torch.equal(c, copies[0])
        assert max_err(c, ref) <= TOL["bf16"]
