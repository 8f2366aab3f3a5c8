"""Calls captured into a HIP graph (torch.cuda.CUDAGraph on a side stream) and replayed.

The workspace of the capture stream is reserved before the capture (a capturing call may
not grow it).  Each replay runs on inputs copied into the captured buffers and writes an
output first filled with a sentinel.  Between replays the program runs eager calls of
its own on the default stream, with its own workspace, and synchronises.  Every replay
must equal the eager call on the same inputs bit for bit: same kernels, same in-kernel
plan, parts merged in a fixed order.  No library call records a memset into the stream,
so nothing here depends on memset nodes in a graph."""
import numpy as np
import pytest

from gpu_util import bf16_dev, f32_dev, i32_dev, need_gpu, u8_dev
from synth import make_decode_case, make_indexer_case, make_sparse_case

pytestmark = pytest.mark.gpu


def check_replays(m, variants, call, make_out, sentinel, ws_bytes, what, replays=6):
    """variants: device-tensor dicts of equal shapes; call(bufs, out) issues one library
    call on torch's current stream."""
    import torch
    bufs = {k: v.clone() for k, v in variants[0].items()}
    out = make_out()
    s = torch.cuda.Stream()
    m.reserve_workspace(ws_bytes, stream=s)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(bufs, out)  # one eager call on the capture stream first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(bufs, out)
    torch.cuda.synchronize()
    for rep in range(replays):
        v = variants[rep % len(variants)]
        for k in bufs:
            bufs[k].copy_(v[k])
        out.fill_(sentinel)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = make_out()
        call(v, want)  # eager, default stream
        torch.cuda.synchronize()
        a = got.view(torch.int16) if got.dtype == torch.bfloat16 else got
        b = want.view(torch.int16) if want.dtype == torch.bfloat16 else want
        assert torch.equal(a, b), f"{what}: replay {rep} differs from the eager call"
    assert m.check_device_errors() == 0
    print(f"[graph] {what}: {replays} replays equal the eager calls", flush=True)


@pytest.mark.parametrize("num_partitions", [0, 3])
def test_graph_decode(num_partitions):
    import torch
    m = need_gpu()
    lens, H = [1500, 3000, 64, 4096, 1, 2222], 128
    variants = []
    for seed in (61, 62, 63):
        c = make_decode_case(seed, lens, H, 64, name="graph-dec")
        variants.append({"q": bf16_dev(c.q), "off": i32_dev(c.input_row_offsets), "pt": i32_dev(c.page_table),
                         "lens": i32_dev(c.cache_lens), "cache": bf16_dev(c.latent_cache)})
    T, scale = c.total_q, c.scale

    def call(b, out):
        m.decode_paged(b["q"], b["off"], b["pt"], b["lens"], b["cache"], scale,
                       num_partitions=num_partitions, out=out)

    def make_out():
        return torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")

    ws = m.decode_workspace_bytes(T, H, num_partitions)
    check_replays(m, variants, call, make_out, float("nan"), ws, f"dense decode num_partitions={num_partitions}")


def test_graph_sparse_decode():
    import torch
    m = need_gpu()
    variants = []
    for seed in (71, 72, 73):
        c = make_sparse_case(seed, 8, 128, 4096, 64, (1, 2048), 2048, name="graph-sparse")
        variants.append({"q": u8_dev(c.q8), "qs": f32_dev(c.q_scale), "off": i32_dev(c.input_row_offsets),
                         "cache": u8_dev(c.cache8), "cs": f32_dev(c.cache_scale), "idx": i32_dev(c.d_indices),
                         "tk": i32_dev(c.topk_lengths)})
    T, H, scale = c.total_q, 128, c.scale

    def call(b, out):
        m.decode_paged_sparse(b["q"], b["qs"], b["off"], b["cache"], b["cs"], b["idx"], b["tk"], scale, out=out)

    def make_out():
        return torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")

    ws = m.decode_workspace_bytes(T, H, 0)
    check_replays(m, variants, call, make_out, float("nan"), ws, "sparse decode")


def test_graph_indexer():
    import torch
    m = need_gpu()
    lens, top_k = [3000, 16384, 700], 1024
    variants = []
    for seed in (81, 82, 83):
        c = make_indexer_case(seed, lens, 16, 128, 64, top_k, q_per_seq=[1, 2, 1], name="graph-idx")
        variants.append({"q": u8_dev(c.q8), "qs": f32_dev(c.q_s), "off": i32_dev(c.input_row_offsets),
                         "pt": i32_dev(c.page_table), "lens": i32_dev(c.cache_lens), "k": u8_dev(c.k8),
                         "ks": f32_dev(c.k_scale)})
    T = c.total_q

    def call(b, out):
        m.indexer_paged_fp8(b["q"], b["qs"], b["off"], b["pt"], b["lens"], b["k"], b["ks"], top_k, out=out)

    def make_out():
        return torch.empty(T, top_k, dtype=torch.int32, device="cuda")

    ws = m.indexer_workspace_bytes(T, c.page_table.shape[1], c.page_size)
    check_replays(m, variants, call, make_out, -7, ws, "indexer")


def test_graph_survives_workspace_growth():
    """A graph captured on a stream keeps replaying correctly after an eager call on the
    same stream has grown that stream's workspace: the outgrown buffer is retired, not
    freed (generic_flare_mla_decode_kv_cache_ragged, Args num_partitions_in: the
    capturable-graph path)."""
    import torch
    m = need_gpu()
    lens, H = [1500, 3000, 64, 4096, 1, 2222], 128
    c = make_decode_case(64, lens, H, 64, name="graph-grow")
    b = {"q": bf16_dev(c.q), "off": i32_dev(c.input_row_offsets), "pt": i32_dev(c.page_table),
         "lens": i32_dev(c.cache_lens), "cache": bf16_dev(c.latent_cache)}
    T = c.total_q

    def call(out, parts):
        m.decode_paged(b["q"], b["off"], b["pt"], b["lens"], b["cache"], c.scale, num_partitions=parts, out=out)

    want = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    call(want, 0)  # eager, default stream
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    out = torch.empty_like(want)
    m.reserve_workspace(m.decode_workspace_bytes(T, H, 0), stream=s)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out, 0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out, 0)
    torch.cuda.synchronize()
    # an eager call on the capture stream that needs more than twice the reserved slots
    big_parts = 200
    assert m.decode_workspace_bytes(T, H, big_parts) > 2 * m.decode_workspace_bytes(T, H, 0)
    other = torch.empty_like(want)
    with torch.cuda.stream(s):
        call(other, big_parts)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep} after growth differs"
        with torch.cuda.stream(s):
            call(other, big_parts)
        torch.cuda.synchronize()
    assert m.check_device_errors(stream=s) == 0
    print("[graph] 3 replays after the capture stream's workspace grew equal the eager call", flush=True)
