"""pkv_decode_noalloc (callers that cannot allocate) against pkv_decode with a
caller workspace: the same kernels, so the outputs must be equal bit for
bit, and both within the bars of the fp64 oracle.  Two calls in a row share
the library's scratch, the second with a smaller input; a call beyond the
scratch is refused on the host."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import TOL, decode_state, max_err, run_decode, say

pytestmark = pytest.mark.gpu


def _noalloc(cache, q, tab, lens, mx, scale, out_dtype=torch.float32, num_splits=0):
    out = torch.full(tuple(q.shape), float("nan"), dtype=out_dtype, device=q.device)
    pkv.decode_noalloc(q, cache.k_cache, cache.v_cache, tab, lens, scale, out, cache.desc, mx,
                       num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def _case(batch, num_splits=0):
    say(f"[noalloc] {batch.name} B={batch.B} maxL={int(batch.lens.max())} splits={num_splits}")
    cache, q, tab, lens, mx = decode_state(batch)
    ref_gpu = run_decode(cache, q, tab, lens, mx, batch.shape.scale, num_splits=num_splits)
    got = _noalloc(cache, q, tab, lens, mx, batch.shape.scale, num_splits=num_splits)
    assert torch.equal(got, ref_gpu)
    ref = oracle.decode(batch.q, batch.k, batch.v, batch.lens, batch.shape.scale)
    err = max_err(got, ref)
    say(f"  bitwise equal to pkv_decode; max abs err vs oracle {err:.3e}")
    assert err <= TOL[batch.shape.dtype], err


def test_two_calls_second_smaller():
    # The Llama-70B-shaped batch (32 sequences, 512-4096 tokens), then the
    # tiny fp32 batch (4 sequences, head_dim 64) on the same scratch.
    _case(synth.cfg2())
    _case(synth.cfg1())


def test_forced_splits_and_ragged_lengths():
    # Many pieces per sequence (partials in every piece slot), then fewer.
    b = synth.custom_decode(901, [1, 17, 300, 1000, 2500], Hq=16, Hkv=2, D=128, dtype="bf16",
                            block_size=16)
    _case(b, num_splits=200)
    _case(synth.custom_decode(902, [5, 40], Hq=4, Hkv=1, D=64, dtype="f32", block_size=32),
          num_splits=3)


def test_beyond_scratch_is_refused():
    b = synth.custom_decode(903, [16] * 600, Hq=64, Hkv=8, D=128, dtype="bf16", block_size=16)
    cache, q, tab, lens, mx = decode_state(b)
    out = torch.zeros(tuple(q.shape), dtype=torch.float32, device=q.device)
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_noalloc(q, cache.k_cache, cache.v_cache, tab, lens, b.shape.scale, out,
                           cache.desc, mx)
    assert e.value.code == pkv.EINVAL
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
