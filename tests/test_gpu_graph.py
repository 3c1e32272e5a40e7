"""The decode step and the chunked prefill under HIP graph capture: the
fused step over 16-bit and E4M3 caches, with a prefix shared by the whole
batch, and in its no-allocation form, and the prefill over 16-bit and E4M3
caches.

A serving loop replays a captured step instead of launching its kernels one
by one.  The library allocates nothing, records no memset, and takes the
caller's stream and workspace, so its launches can be captured.  Each graph
here is replayed several times, with new query values copied into its
static inputs and with eager work between the replays; every replay must
equal the same call made eagerly on the same inputs, bit for bit (outputs
and caches)."""
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


def filled_caches(w, tdt):
    ksh, vsh = w.cache_shapes()
    kc = torch.zeros(ksh, dtype=tdt, device=DEV)
    vc = torch.zeros(vsh, dtype=tdt, device=DEV)
    k, v, s = w.write_batch("hist")
    B.paged_kv_write(dev_bits(k, tdt), dev_bits(v, tdt), torch.from_numpy(s).to(DEV), kc, vc)
    return kc, vc


def test_fused_decode_step_graph_replay():
    w = W.build("graph", list(np.random.default_rng(5).integers(1, 700, size=24)),
                num_heads=16, num_kv_heads=4, head_dim=128, block_size=16, dtype=W.BF16,
                seed=17)
    tdt = torch.bfloat16
    nk, nv, _ = w.write_batch("new")
    k_new, v_new = dev_bits(nk, tdt), dev_bits(nv, tdt)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    need = B.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                             w.max_blocks_per_seq, w.block_size)
    ws_graph = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_eager = torch.empty(need, dtype=torch.uint8, device=DEV)
    kc_g, vc_g = filled_caches(w, tdt)
    kc_e, vc_e = filled_caches(w, tdt)
    q = dev_bits(w.q, tdt)
    out = torch.empty_like(q)

    def step(o, kc, vc, ws):
        B.paged_attention_decode_append(o, q, k_new, v_new, kc, vc, bt, cl, w.scale,
                                        w.block_size, w.num_kv_heads, workspace_tensor=ws)

    step(out, kc_g, vc_g, ws_graph)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out, kc_g, vc_g, ws_graph)
    gen = torch.Generator(device="cpu").manual_seed(3)
    for r in range(4):
        say(f"graph replay {r}")
        q.copy_(torch.randn(q.shape, generator=gen).to(tdt).to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        step(ref, kc_e, vc_e, ws_eager)  # eager work between replays, and the reference
        junk = torch.empty_like(out)
        step(junk, kc_e, vc_e, ws_graph)  # eager use of the graph's own workspace
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        assert torch.equal(kc_g.view(torch.int16), kc_e.view(torch.int16))
        assert torch.equal(vc_g.view(torch.int16), vc_e.view(torch.int16))


@pytest.mark.parametrize("kv8", [False, True], ids=["f16", "e4m3"])
def test_prefill_graph_replay(kv8):
    lengths, chunks = [300, 97, 512, 40], [300, 33, 128, 1]
    w = W.build("graphpf", lengths, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                dtype=W.F16, seed=23)
    tdt = torch.float16
    ksh, vsh = w.cache_shapes()
    ct = torch.uint8 if kv8 else tdt
    kc = torch.zeros(ksh, dtype=ct, device=DEV)
    vc = torch.zeros(vsh, dtype=ct, device=DEV)
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        kd, vd, sd = dev_bits(k, tdt), dev_bits(v, tdt), torch.from_numpy(s).to(DEV)
        if kv8:
            B.paged_kv_write_fp8(kd, vd, sd, kc, vc, 0.02, 0.03)
        else:
            B.paged_kv_write(kd, vd, sd, kc, vc)
    qs = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    rows = int(sum(chunks))
    q = torch.zeros(rows, 8, 128, dtype=tdt, device=DEV)
    out = torch.empty_like(q)

    def call(o):
        if kv8:
            B.paged_attention_prefill_fp8(o, q, kc, vc, bt, cl, qs, w.scale, 0.02, 0.03, 16, 2,
                                          max(chunks))
        else:
            B.paged_attention_prefill(o, q, kc, vc, bt, cl, qs, w.scale, 16, 2, max(chunks))

    call(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    gen = torch.Generator(device="cpu").manual_seed(4)
    for r in range(4):
        say(f"prefill graph replay {r} kv8={kv8}")
        q.copy_(torch.randn(q.shape, generator=gen).to(tdt).to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        call(ref)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {r}"


def check_replays(tag, q, out, graph_call, eager_call, graph_ws_eager, caches_g, caches_e):
    """Capture graph_call() (writes out and caches_g), then replay it four
    times with new query values.  After each replay: eager_call() returns the
    same step made eagerly on caches_e, which must equal the replay bit for
    bit (output and caches); graph_ws_eager() then uses the graph's own
    workspace eagerly on caches_e, as a serving loop's other calls may."""
    graph_call()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_call()
    gen = torch.Generator(device="cpu").manual_seed(3)
    for r in range(4):
        say(f"{tag} graph replay {r}")
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype).to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = eager_call()
        graph_ws_eager()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{tag} replay {r}"
        for a, b in zip(caches_g, caches_e):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{tag} caches {r}"


def fp8_caches(w, tdt, ks, vs):
    ksh, vsh = w.cache_shapes()
    kc = torch.zeros(ksh, dtype=torch.uint8, device=DEV)
    vc = torch.zeros(vsh, dtype=torch.uint8, device=DEV)
    k, v, s = w.write_batch("hist")
    B.paged_kv_write_fp8(dev_bits(k, tdt), dev_bits(v, tdt), torch.from_numpy(s).to(DEV), kc,
                         vc, ks, vs)
    return kc, vc


def test_fused_decode_step_e4m3_graph_replay():
    """The fused step over E4M3 caches (quantising append, decode) captured."""
    w = W.build("graph8", list(np.random.default_rng(6).integers(1, 700, size=24)),
                num_heads=16, num_kv_heads=4, head_dim=128, block_size=16, dtype=W.BF16,
                seed=18)
    tdt = torch.bfloat16
    nk, nv, _ = w.write_batch("new")
    k_new, v_new = dev_bits(nk, tdt), dev_bits(nv, tdt)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    need = B.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                             w.max_blocks_per_seq, w.block_size)
    ws_g = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_e = torch.empty(need, dtype=torch.uint8, device=DEV)
    kc_g, vc_g = fp8_caches(w, tdt, 0.02, 0.03)
    kc_e, vc_e = fp8_caches(w, tdt, 0.02, 0.03)
    q = dev_bits(w.q, tdt)
    out = torch.empty_like(q)

    def step(o, kc, vc, ws):
        B.paged_attention_decode_append(o, q, k_new, v_new, kc, vc, bt, cl, w.scale,
                                        w.block_size, w.num_kv_heads, k_scale=0.02,
                                        v_scale=0.03, workspace_tensor=ws)
        return o

    check_replays("e4m3", q, out, lambda: step(out, kc_g, vc_g, ws_g),
                  lambda: step(torch.empty_like(out), kc_e, vc_e, ws_e),
                  lambda: step(torch.empty_like(out), kc_e, vc_e, ws_g),
                  (kc_g, vc_g), (kc_e, vc_e))


def test_shared_prefix_step_graph_replay():
    """The fused step with a prefix of 20 blocks shared by every sequence
    (the shared path's two kinds of wavefront and its merge) captured."""
    g0 = np.random.default_rng(7)
    w = W.build("graphsh", list(320 + g0.integers(1, 300, size=24)), num_heads=16,
                num_kv_heads=4, head_dim=128, block_size=16, dtype=W.BF16, seed=19,
                shared_prefix_tokens=320)
    tdt = torch.bfloat16
    sb = 320 // 16
    nk, nv, _ = w.write_batch("new")
    k_new, v_new = dev_bits(nk, tdt), dev_bits(nv, tdt)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    need = B.workspace_bytes_shared(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                    w.max_blocks_per_seq, w.block_size, sb, 0)
    ws_g = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_e = torch.empty(need, dtype=torch.uint8, device=DEV)
    kc_g, vc_g = filled_caches(w, tdt)
    kc_e, vc_e = filled_caches(w, tdt)
    q = dev_bits(w.q, tdt)
    out = torch.empty_like(q)

    def step(o, kc, vc, ws):
        B.paged_attention_decode_shared(o, q, kc, vc, bt, cl, w.scale, w.block_size,
                                        w.num_kv_heads, sb, k_new=k_new, v_new=v_new,
                                        workspace_tensor=ws)
        return o

    check_replays("shared", q, out, lambda: step(out, kc_g, vc_g, ws_g),
                  lambda: step(torch.empty_like(out), kc_e, vc_e, ws_e),
                  lambda: step(torch.empty_like(out), kc_e, vc_e, ws_g),
                  (kc_g, vc_g), (kc_e, vc_e))


def test_noalloc_step_graph_replay():
    """The no-allocation fused step (its workspace is the library's own
    device array) captured; each replay equals the step with a caller's
    workspace, and an eager no-allocation call runs between replays."""
    w = W.build("graphna", list(np.random.default_rng(8).integers(1, 700, size=24)),
                num_heads=16, num_kv_heads=4, head_dim=128, block_size=16, dtype=W.BF16,
                seed=20)
    tdt = torch.bfloat16
    nk, nv, _ = w.write_batch("new")
    k_new, v_new = dev_bits(nk, tdt), dev_bits(nv, tdt)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    need = B.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                             w.max_blocks_per_seq, w.block_size)
    ws_e = torch.empty(need, dtype=torch.uint8, device=DEV)
    kc_g, vc_g = filled_caches(w, tdt)
    kc_e, vc_e = filled_caches(w, tdt)
    q = dev_bits(w.q, tdt)
    out = torch.empty_like(q)

    def noalloc(o, kc, vc):
        B.paged_attention_decode_append_noalloc(o, q, k_new, v_new, kc, vc, bt, cl, w.scale,
                                                w.block_size, w.num_kv_heads)
        return o

    def with_ws(o, kc, vc):
        B.paged_attention_decode_append(o, q, k_new, v_new, kc, vc, bt, cl, w.scale,
                                        w.block_size, w.num_kv_heads, workspace_tensor=ws_e)
        return o

    check_replays("noalloc", q, out, lambda: noalloc(out, kc_g, vc_g),
                  lambda: with_ws(torch.empty_like(out), kc_e, vc_e),
                  lambda: noalloc(torch.empty_like(out), kc_e, vc_e),
                  (kc_g, vc_g), (kc_e, vc_e))
