"""Per-step metadata staged in pinned host memory and copied asynchronously
(block tables, context lengths, slots; "LLM Inference: KV Cache, Batching &
Scheduling", "PagedAttention and vLLM": the host keeps the logical-to-physical
map and it changes every step).  The staged arrays must equal the ones the
synchronous path builds, and a decode step run on them must give the same
output bit for bit, over more steps than the ring has buffers."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indirected_amd as pkv
import synth
from harness import say
from paged_kv_cache_indirected_amd.paged import PagedCache, StepMetadata, to_device_rows

pytestmark = pytest.mark.gpu


def test_staged_metadata_equals_synchronous_and_decodes_bitwise():
    b = synth.custom_decode(950, [1, 15, 16, 17, 200, 700], Hq=16, Hkv=2, D=128, dtype="bf16",
                            block_size=16)
    sh = b.shape
    st = b.seq_start()
    ids = list(range(b.B))
    steps, depth = 9, 3
    stride = int((b.lens.max() + steps + sh.block_size) // sh.block_size) + 1
    ca = PagedCache(b.pool_blocks + 64, sh.Hkv, sh.block_size, sh.D, pkv.BF16, pool_seed=7)
    cb = PagedCache(b.pool_blocks + 64, sh.Hkv, sh.block_size, sh.D, pkv.BF16, pool_seed=7)
    for c in (ca, cb):
        c.add_sequences(ids, b.lens, b.k, b.v)
    md = StepMetadata(b.B, stride, depth=depth)
    ws = torch.empty(pkv.decode_workspace_bytes(b.B, sh.Hq, stride * sh.block_size, ca.desc),
                     dtype=torch.uint8, device="cuda")
    g = np.random.default_rng(5)
    for step in range(steps):
        say(f"[metadata] step {step}")
        kn = synth.normal(g, (b.B, sh.Hkv, sh.D), "bf16")
        vn = synth.normal(g, (b.B, sh.Hkv, sh.D), "bf16")
        qn = to_device_rows(synth.normal(g, (b.B, sh.Hq, sh.D), "bf16"), pkv.BF16, "cuda")
        kd, vd = to_device_rows(kn, pkv.BF16, "cuda"), to_device_rows(vn, pkv.BF16, "cuda")
        # synchronous path
        slots_a = torch.from_numpy(ca.seqs.append_batch(ids)).to("cuda")
        tab_a, lens_a, mx_a = ca.tables(ids, stride)
        # staged path (pinned ring, one async copy)
        tab_b, lens_b, slots_b, mx_b = md.stage(cb.seqs, ids)
        assert mx_a == mx_b
        outs = []
        for c, tab, lens, slots, mx in ((ca, tab_a, lens_a, slots_a, mx_a),
                                        (cb, tab_b, lens_b, slots_b, mx_b)):
            out = torch.full((b.B, sh.Hq, sh.D), float("nan"), device="cuda")
            pkv.append_decode(kd, vd, slots, qn, c.k_cache, c.v_cache, tab, lens, sh.scale, out,
                              c.desc, mx, workspace=ws)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(tab_a, tab_b) and torch.equal(lens_a, lens_b)
        assert torch.equal(slots_a, slots_b)
        assert torch.equal(outs[0], outs[1])
        assert torch.equal(ca.k_cache.view(torch.int16), cb.k_cache.view(torch.int16))
