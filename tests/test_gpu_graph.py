"""The decode steps under HIP graph capture (needs an MI355X): each step is
captured once on torch's capture stream and replayed several times, with
eager work and synchronizations between the replays; every replay must give
the eager result bit for bit (the library enqueues only kernels on the
caller's stream: no memset, allocation or synchronization inside a step)."""
import pytest
import torch

import decode_attention_paged_append_amd as pa
import workloads as W
from gpu_cases import dev
from test_gpu_kernels import make, to_dev
import test_gpu_quant_step as QS

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8).clone()


def check_graph(run, out, caches, replays=3):
    """run() enqueues one step writing out and appending to caches (the same
    bytes every time).  out is overwritten between the replays."""
    run()
    torch.cuda.synchronize()
    eager = [bits(t) for t in (out, *caches)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the capture, as torch advises
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for i in range(replays):
        out.view(torch.uint8).fill_(0xA5)   # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip((out, *caches), eager):
            assert torch.equal(bits(t), e), f"replay {i} differs from the eager step"


def test_graph_fused_step_f16_partitions():
    """Vector-ALU kernel, several partitions, fused append, then the merge."""
    hq = hkv = 8
    shape, lay, case = make("f16", hq, hkv, 128, 16, [900, 17, 4000, 1], seed=51,
                            poison_new=True)
    q, kc, vc, kn, vn, bt, ctx = to_dev(case.q, case.k_cache, case.v_cache, case.k_new,
                                        case.v_new, lay.block_tables, lay.context_lens)
    out = torch.empty_like(q)
    ws = torch.empty(max(pa.decode_workspace_bytes(kc, 4, hq, lay.max_blocks), 256),
                     dtype=torch.uint8, device=dev())
    print("graph: f16 fused step", flush=True)
    check_graph(lambda: pa.decode_step(q, kn, vn, kc, vc, bt, ctx, shape.scale, out, ws),
                out, [kc, vc])


def test_graph_paired_step_bf16():
    """Matrix-core kernel, paired plan (one partition over the table)."""
    hq, hkv, bs = 64, 8, 16
    ctx = [int(x) for x in torch.randint(1, 600, (65,), generator=W.generator(3))]
    shape, lay, case = make("bf16", hq, hkv, 128, bs, ctx, seed=52, poison_new=True)
    q, kc, vc, kn, vn, bt, ctx_t = to_dev(case.q, case.k_cache, case.v_cache, case.k_new,
                                          case.v_new, lay.block_tables, lay.context_lens)
    out = torch.empty_like(q)
    print("graph: bf16 paired step", flush=True)
    check_graph(lambda: pa.decode_step_partitions(q, kn, vn, kc, vc, bt, ctx_t, shape.scale,
                                                  out, lay.max_blocks * bs, None),
                out, [kc, vc])


@pytest.mark.parametrize("fmt", ["i8", "fp8", "i4"])
def test_graph_quant_step(fmt):
    """Quantizing append fused into the attention launch, library plan."""
    hq, hkv, d, bs = 32, 8, 128, 16
    shape, lay, case, start, _ = QS.setup(fmt, hq, hkv, d, bs, [700, 3000, 1, 64], seed=53)
    pools = [QS.to_gpu(fmt, a) for a in start]
    q, kn, vn, bt, ctx = to_dev(case.q, case.k_new, case.v_new, lay.block_tables,
                                lay.context_lens)
    out = torch.empty_like(q)
    desc = pa.int4_desc(pools[0]) if fmt == "i4" else pa.CacheDesc.of(pools[0])
    ws = torch.empty(max(pa.decode_workspace_bytes(desc, 4, hq, lay.max_blocks), 256),
                     dtype=torch.uint8, device=dev())
    print(f"graph: {fmt} quantized step", flush=True)
    check_graph(lambda: pa.decode_step_quant(q, kn, vn, *pools, bt, ctx, shape.scale, out, ws,
                                             int4=fmt == "i4"),
                out, pools)


def test_graph_window_step():
    """Windowed step (fused append, merge inside) on the matrix cores."""
    hq, hkv, bs, window = 32, 8, 16, 1000
    shape, lay, case = make("f16", hq, hkv, 128, bs, [3000, 999, 1001, 40], seed=54,
                            poison_new=True)
    q, kc, vc, kn, vn, bt, ctx = to_dev(case.q, case.k_cache, case.v_cache, case.k_new,
                                        case.v_new, lay.block_tables, lay.context_lens)
    out = torch.empty_like(q)
    ws = torch.empty(max(pa.decode_window_workspace_bytes(kc, 4, hq, lay.max_blocks, window),
                         256), dtype=torch.uint8, device=dev())
    print("graph: f16 window step", flush=True)
    check_graph(lambda: pa.decode_step_window(q, kn, vn, kc, vc, bt, ctx, shape.scale, window,
                                              out, workspace=ws),
                out, [kc, vc])
