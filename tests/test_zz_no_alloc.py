"""sv_verify_batch_noalloc (GPU, through the C ABI): the entry point that allocates nothing and
runs on the library's per-GPU scratch array gives exactly what sv_verify_batch gives with a
caller's workspace, on two calls in a row (the second smaller), and matches the oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

import lossless_draft_verification_sv_amd as sv  # noqa: E402
from tests.gpu_util import check_sample_parity, run_sample, say, to_dev  # noqa: E402
from workloads import BATCHED, TINY, generate  # noqa: E402


def run_noalloc(inp):
    lib = sv.load_library()
    w = inp.workload
    dev = torch.device("cuda:0")
    T, D = to_dev(inp.target), to_dev(inp.draft)
    x, u, r = to_dev(inp.tokens), to_dev(inp.uniforms), to_dev(inp.residual)
    nd = None if inp.num_draft is None else to_dev(inp.num_draft)
    acc = torch.full((w.B,), -7, dtype=torch.int32, device=dev)
    com = torch.full((w.B, w.K + 1), -7, dtype=torch.int32, device=dev)
    tp = torch.full((w.B, w.K), -7.0, dtype=torch.float32, device=dev)
    dp = torch.full((w.B, w.K), -7.0, dtype=torch.float32, device=dev)
    code = sv.SV_DTYPE_BF16 if w.dtype == "bf16" else sv.SV_DTYPE_F32
    st = lib.sv_verify_batch_noalloc(T.data_ptr(), D.data_ptr(), code, w.B, w.K, w.V,
                                     w.temperature, x.data_ptr(),
                                     None if nd is None else nd.data_ptr(), u.data_ptr(),
                                     r.data_ptr(), acc.data_ptr(), com.data_ptr(), tp.data_ptr(),
                                     dp.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, sv.sv_last_error()
    torch.cuda.synchronize()
    return acc.cpu().numpy(), com.cpu().numpy(), tp.cpu().numpy(), dp.cpu().numpy()


def same_as_workspace_call(inp, name):
    w = inp.workload
    got = run_noalloc(inp)
    ref = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                     w.temperature, inp.num_draft)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), name
    check_sample_parity(name, inp.target, inp.draft, w.dtype, inp.tokens, inp.uniforms,
                        inp.residual, w.temperature, inp.num_draft)
    say(f"[gpu] noalloc {name}: identical to sv_verify_batch with a workspace")


def test_noalloc_two_calls_second_smaller():
    big = generate(BATCHED.replace(name="noalloc_big", B=12, seed=6101))
    small = generate(TINY.replace(name="noalloc_small", B=3, K=3, V=5000, seed=6102))
    same_as_workspace_call(big, "big")
    same_as_workspace_call(small, "small")
    same_as_workspace_call(big, "big again")


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    lib = sv.load_library()
    need = int(lib.sv_workspace_bytes(4096, 64, 151936))
    assert need > 16 << 20
    st = lib.sv_verify_batch_noalloc(16, 16, sv.SV_DTYPE_BF16, 4096, 64, 151936, 1.0, 16, None, 16,
                                     16, 16, 16, 16, None, None)
    assert st == sv.SV_ERR_UNSUPPORTED and "scratch" in sv.sv_last_error()


def test_noalloc_captured_graph_replays():
    """One sv_verify_batch_noalloc call captured into a HIP graph (torch.cuda.CUDAGraph) and
    replayed for several batches copied into its input buffers, with eager work and a device
    synchronisation between the replays: every replay gives exactly what sv_verify_batch gives
    with a workspace on the same batch (the call clears its scratch words and hands off under
    one fixed tag, so a replay never takes an earlier replay's words for its own)."""
    lib = sv.load_library()
    batches = [generate(BATCHED.replace(name=f"noalloc_graph_{i}", B=6, V=30000, seed=6200 + i))
               for i in range(3)]
    w = batches[0].workload
    dev = torch.device("cuda:0")
    T, D = to_dev(batches[0].target), to_dev(batches[0].draft)
    x, u, r = to_dev(batches[0].tokens), to_dev(batches[0].uniforms), to_dev(batches[0].residual)
    acc = torch.empty((w.B,), dtype=torch.int32, device=dev)
    com = torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev)
    tp = torch.empty((w.B, w.K), dtype=torch.float32, device=dev)
    dp = torch.empty((w.B, w.K), dtype=torch.float32, device=dev)
    code = sv.SV_DTYPE_BF16 if w.dtype == "bf16" else sv.SV_DTYPE_F32

    def call():
        st = lib.sv_verify_batch_noalloc(T.data_ptr(), D.data_ptr(), code, w.B, w.K, w.V,
                                         w.temperature, x.data_ptr(), None, u.data_ptr(),
                                         r.data_ptr(), acc.data_ptr(), com.data_ptr(),
                                         tp.data_ptr(), dp.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
        assert st == 0, sv.sv_last_error()

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # eager first calls: the scratch address and occupancy are looked up here
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i, inp in enumerate(batches + batches[:1]):
        T.copy_(to_dev(inp.target))
        D.copy_(to_dev(inp.draft))
        x.copy_(to_dev(inp.tokens))
        u.copy_(to_dev(inp.uniforms))
        r.copy_(to_dev(inp.residual))
        for out in (acc, com, tp, dp):
            out.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (acc.cpu().numpy(), com.cpu().numpy(), tp.cpu().numpy(), dp.cpu().numpy())
        ref = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                         w.temperature)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), i
        say(f"[gpu] noalloc graph replay {i}: identical to sv_verify_batch with a workspace")
