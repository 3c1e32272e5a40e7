"""Decode calls on two streams at once, through the binding's cached
workspaces.

The binding keeps one workspace per (device, stream): a decode writes its
partial results there and reads them back in its second launch on the same
stream, so calls on different streams must not share one.  Two workloads
of different shapes are decoded alternately on two side streams (default
priority), eight times each with no synchronisation between them; every
output must equal the same call made alone on the default stream, bit for
bit.
"""
import numpy as np
import pytest
import torch

from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def dev_bits(bits, tdt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(tdt)


def setup(w, tdt):
    ksh, vsh = w.cache_shapes()
    kc = torch.zeros(ksh, dtype=tdt, device=DEV)
    vc = torch.zeros(vsh, dtype=tdt, device=DEV)
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        B.paged_kv_write(dev_bits(k, tdt), dev_bits(v, tdt), torch.from_numpy(s).to(DEV), kc, vc)
    return dict(q=dev_bits(w.q, tdt), kc=kc, vc=vc, bt=torch.from_numpy(w.block_tables).to(DEV),
                cl=torch.from_numpy(w.context_lens).to(DEV))


def decode(w, d):
    out = torch.empty_like(d["q"])
    B.paged_attention_decode(out, d["q"], d["kc"], d["vc"], d["bt"], d["cl"], w.scale,
                             w.block_size, w.num_kv_heads)
    return out


def test_two_streams_keep_their_own_workspaces():
    g = np.random.default_rng(31)
    wa = W.build("streamA", list(g.integers(1, 900, size=40)), num_heads=32, num_kv_heads=8,
                 head_dim=128, block_size=16, dtype=W.BF16, seed=41)
    wb = W.build("streamB", list(g.integers(1, 400, size=24)), num_heads=16, num_kv_heads=4,
                 head_dim=64, block_size=8, dtype=W.BF16, seed=42)
    da, db = setup(wa, torch.bfloat16), setup(wb, torch.bfloat16)
    ref_a, ref_b = decode(wa, da), decode(wb, db)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for r in range(8):
        with torch.cuda.stream(s1):
            outs.append(("a", r, decode(wa, da)))
        with torch.cuda.stream(s2):
            outs.append(("b", r, decode(wb, db)))
    torch.cuda.synchronize()
    for which, r, o in outs:
        ref = ref_a if which == "a" else ref_b
        say(f"stream {which} call {r}")
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"{which} call {r}"
