"""The no-allocation fused step (paged_attention_decode_append_noalloc)
against the step with a caller workspace (paged_attention_decode_append).

Two calls in a row share the library's fixed scratch array, the second with
a smaller input, so it runs over the bytes the first left behind.  Each call
must give the outputs and caches of paged_attention_decode_append bit for bit
(the same kernels run; only the workspace differs), the caches must equal
the oracle's appends and the outputs must meet
|gpu - oracle| <= 2e-3 + 1e-2 * |oracle|.  torch's allocator must not grow
during a call.
"""
import numpy as np
import pytest
import torch

import oracle
from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {W.F16: torch.float16, W.BF16: torch.bfloat16}
ATOL, RTOL = 2e-3, 1e-2
KS, VS = 0.02, 0.03


def say(msg):
    print(msg, flush=True)


def dev_bits(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(TD[dtype])


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == W.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Step:
    """Caches holding one workload's history, and the fused step's inputs."""

    def __init__(self, w, fp8):
        self.w, self.fp8 = w, fp8
        ks, vs = w.cache_shapes()
        if fp8:
            self.kc0 = torch.full(ks, W.FP8_NAN, dtype=torch.uint8, device=DEV)
            self.vc0 = torch.full(vs, W.FP8_NAN, dtype=torch.uint8, device=DEV)
        else:
            nan = int(np.array([W.NAN_BITS[w.dtype]], np.uint16).view(np.int16)[0])
            self.kc0 = torch.full(ks, nan, dtype=torch.int16, device=DEV).view(TD[w.dtype])
            self.vc0 = torch.full(vs, nan, dtype=torch.int16, device=DEV).view(TD[w.dtype])
        k, v, s = w.write_batch("hist")
        if fp8:
            B.paged_kv_write_fp8(dev_bits(k, w.dtype), dev_bits(v, w.dtype),
                                 torch.from_numpy(s).to(DEV), self.kc0, self.vc0, KS, VS)
        else:
            B.paged_kv_write(dev_bits(k, w.dtype), dev_bits(v, w.dtype),
                             torch.from_numpy(s).to(DEV), self.kc0, self.vc0)
        kn, vn, _ = w.write_batch("new")
        self.kn, self.vn = dev_bits(kn, w.dtype), dev_bits(vn, w.dtype)
        self.q = dev_bits(w.q, w.dtype)
        self.bt = torch.from_numpy(w.block_tables).to(DEV)
        self.cl = torch.from_numpy(w.context_lens).to(DEV)
        torch.cuda.synchronize()

    def run(self, fn):
        w = self.w
        kc, vc = self.kc0.clone(), self.vc0.clone()
        out = torch.full_like(self.q, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        fn(out, self.q, self.kn, self.vn, kc, vc, self.bt, self.cl, w.scale, w.block_size,
           w.num_kv_heads, k_scale=KS if self.fp8 else None, v_scale=VS if self.fp8 else None)
        grew = torch.cuda.memory_allocated() - before
        torch.cuda.synchronize()
        if self.fp8:
            return host_bits(out), kc.cpu().numpy(), vc.cpu().numpy(), grew
        return host_bits(out), host_bits(kc), host_bits(vc), grew

    def check_oracle(self, out, kc, vc):
        w = self.w
        rk, rv = w.nan_caches_fp8() if self.fp8 else w.nan_caches()
        for which in ("hist", "new"):
            k, v, s = w.write_batch(which)
            if self.fp8:
                oracle.kv_write_fp8(k, v, s, rk, rv, w.block_size, w.dtype, KS, VS)
            else:
                oracle.kv_write(k, v, s, rk, rv, w.block_size)
        assert np.array_equal(kc, rk) and np.array_equal(vc, rv), "caches differ from oracle"
        rows = oracle.all_rows(w.num_seqs, w.num_heads)
        if self.fp8:
            ref = oracle.decode_fp8_rows(rows, w.q, rk, rv, w.block_tables, w.context_lens,
                                         w.scale, w.block_size, w.dtype, KS, VS,
                                         threads=oracle.host_threads())
        else:
            ref = oracle.decode_rows(rows, w.q, rk, rv, w.block_tables, w.context_lens,
                                     w.scale, w.block_size, w.dtype,
                                     threads=oracle.host_threads())
        err = np.abs(f64(out, w.dtype) - ref.reshape(out.shape))
        assert np.all(err <= ATOL + RTOL * np.abs(ref.reshape(out.shape)))
        return err.max()


def _workloads():
    big = W.llama8b()
    small = W.build("noalloc_small", [1, 17, 300, 33, 16, 5, 129], num_heads=8, num_kv_heads=2,
                    head_dim=64, block_size=8, dtype=W.F16, seed=515)
    return big, small


@pytest.mark.parametrize("fp8", [False, True], ids=["16bit", "e4m3"])
def test_noalloc_matches_workspace_call(fp8):
    big, small = _workloads()
    # the second call's workspace is smaller than the first's
    assert (B.workspace_bytes(small.num_seqs, small.num_heads, small.num_kv_heads,
                              small.head_dim, small.max_blocks_per_seq, small.block_size) <
            B.workspace_bytes(big.num_seqs, big.num_heads, big.num_kv_heads, big.head_dim,
                              big.max_blocks_per_seq, big.block_size))
    for i, w in enumerate((big, small)):
        say(f"noalloc call {i + 1}: {w.name} B={w.num_seqs} fp8={fp8}")
        st = Step(w, fp8)
        got = st.run(B.paged_attention_decode_append_noalloc)
        ref = st.run(B.paged_attention_decode_append)
        assert got[3] == 0, f"torch's allocator grew by {got[3]} bytes during the call"
        for a, b in zip(got[:3], ref[:3]):
            assert np.array_equal(a, b), "differs from paged_attention_decode_append"
        e = st.check_oracle(*got[:3])
        say(f"  bit-identical to the workspace call; max abs error vs oracle {e:.3e}")


def test_noalloc_refuses_oversized():
    """A batch whose workspace exceeds the fixed array raises before any
    launch, and leaves out untouched."""
    w = W.build("noalloc_big", [16] * 512, num_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, dtype=W.BF16, seed=516, max_blocks_per_seq=128)
    assert B.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                             w.max_blocks_per_seq, w.block_size) > B.SCRATCH_BYTES
    st = Step(w, False)
    with pytest.raises(ValueError, match="scratch"):
        st.run(B.paged_attention_decode_append_noalloc)
