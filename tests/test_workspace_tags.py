"""Workspace reuse and call tags on the GPU, through the C ABI.

Every word one work-group hands another inside a launch carries a number of the call (the upper
32 bits). The library draws these from one process-wide counter and zero-fills a workspace
itself on its first tagged call after the counter's low 32 bits wrap, and after a function that
leaves untagged words (the per-position Markov form, top-K) used it. These tests plant words
that would pass for the next call's (the tag it will draw, garbage payloads) and check that the
results still match the oracle; and they run the one-launch Markov head (a cooperative launch)
while another stream keeps a long read kernel on the device.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

import lossless_draft_verification_sv_amd as sv  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from tests.gpu_util import say, to_dev  # noqa: E402
from workloads import BATCHED, generate  # noqa: E402

STALE_PAYLOAD = 0x7F7FFFFF  # the largest finite float: a partial no real row produces


def plant(ws: torch.Tensor, tags) -> None:
    """Fills the workspace with 64-bit words carrying the given tags (cycled) and a garbage
    payload, as an earlier call could have left them."""
    words = ws.view(torch.int64)
    tags = np.asarray(list(tags), dtype=np.int64)
    vals = (tags << 32) | STALE_PAYLOAD
    pattern = torch.from_numpy(np.resize(vals, words.numel())).to(ws.device)
    words.copy_(pattern)
    torch.cuda.synchronize()


def verify_call(lib, inp, ws):
    w = inp.workload
    dev = torch.device("cuda:0")
    T, D = to_dev(inp.target), to_dev(inp.draft)
    x, u, r = to_dev(inp.tokens), to_dev(inp.uniforms), to_dev(inp.residual)
    acc = torch.empty(w.B, dtype=torch.int32, device=dev)
    com = torch.empty(w.B, w.K + 1, dtype=torch.int32, device=dev)
    tp = torch.empty(w.B, w.K, dtype=torch.float32, device=dev)
    code = sv.SV_DTYPE_BF16 if w.dtype == "bf16" else sv.SV_DTYPE_F32
    st = lib.sv_verify_batch(T.data_ptr(), D.data_ptr(), code, w.B, w.K, w.V, w.temperature,
                             x.data_ptr(), None, u.data_ptr(), r.data_ptr(), acc.data_ptr(),
                             com.data_ptr(), tp.data_ptr(), None, ws.data_ptr(), ws.numel(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0, sv.sv_last_error()
    torch.cuda.synchronize()
    return acc.cpu().numpy(), com.cpu().numpy(), tp.cpu().numpy()


def check_verify(inp, out):
    w = inp.workload
    ref = oracle.verify_batch(inp.target, inp.draft, w.dtype, inp.tokens, inp.uniforms,
                              inp.residual, w.temperature)
    acc, com, tp = out
    ok = ~ref.ambiguous
    assert np.array_equal(acc[ok], ref.accepted_len[ok])
    assert np.array_equal(com[ok], ref.committed[ok])
    assert np.max(np.abs(tp - ref.target_prob)) <= 1e-5


def test_verify_across_a_counter_wrap_with_stale_words():
    lib = sv.load_library()
    inp = generate(BATCHED.replace(name="wrap", B=6, K=4, V=20000, seed=5101))
    w = inp.workload
    nbytes = int(lib.sv_workspace_bytes(w.B, w.K, w.V))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    check_verify(inp, verify_call(lib, inp, ws))  # the library has now seen ws
    base = 7 << 32
    # the last tag of a wrap period: the call is the first on ws in that period
    lib.sv_set_call_counter(base - 1)
    plant(ws, [0xFFFFFFFF])
    check_verify(inp, verify_call(lib, inp, ws))
    # the next call skips tag 0 and takes tag 1 of the next period; words stamped 1 from the
    # period before must not pass for its own
    plant(ws, [1])
    check_verify(inp, verify_call(lib, inp, ws))
    # within one period no fill is needed: words of other tags are ignored
    plant(ws, [5, 6, 0xFFFFFFFF])
    check_verify(inp, verify_call(lib, inp, ws))
    say("[gpu] verify across a counter wrap: stale words filled, results match the oracle")


def markov_inputs(B, K, V, R, seed):
    base = workloads.markov_base(B, K, V, "bf16", seed=seed)
    left, right = workloads.markov_factors(V, R, seed=seed + 1)
    anchor = np.random.default_rng(seed + 2).integers(0, V, size=B).astype(np.int32)
    return base, left, right, anchor


def markov_call(lib, base, left, right, anchor, ws, stream=None):
    B, K, V = base.shape
    R = left.shape[1]
    dev = torch.device("cuda:0")
    b, l, r, a = to_dev(base), to_dev(left), to_dev(right), to_dev(anchor)
    tok = torch.empty(B, K, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream() if stream is None else stream
    st = lib.sv_markov_draft(b.data_ptr(), sv.SV_DTYPE_BF16, B, K, V, l.data_ptr(), r.data_ptr(),
                             R, a.data_ptr(), tok.data_ptr(), None, ws.data_ptr(), ws.numel(),
                             s.cuda_stream)
    assert st == 0, sv.sv_last_error()
    return tok


def check_markov(name, tok, base, left, right, anchor):
    tok = tok.cpu().numpy()
    ref, _, amb = oracle.markov_draft(base, "bf16", left, right, anchor)
    assert np.array_equal(tok[~amb], ref[~amb]), name
    say(f"[gpu] markov {name}: {int((~amb).sum())} positions exact")


def test_markov_one_launch_across_a_wrap_and_after_topk_on_one_workspace():
    """The one-launch head (B <= 64, R <= 256) takes 2K + 2 tags per call; the same memory also
    serves top-K (untagged tables) and the per-position form (B > 128, untagged argmaxes)."""
    lib = sv.load_library()
    B, K, V, R = 8, 4, 6000, 64
    base, left, right, anchor = markov_inputs(B, K, V, R, 5201)
    need = max(int(lib.sv_markov_workspace_bytes(B, V)),
               int(lib.sv_markov_topk_workspace_bytes(B, K, V)),
               int(lib.sv_markov_workspace_bytes(130, V)))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    check_markov("first", markov_call(lib, base, left, right, anchor, ws), base, left, right,
                 anchor)
    # across a wrap: the next call skips the tags that would reach past 2^32 and takes the
    # first 2K + 2 of the next period after tag 0
    lib.sv_set_call_counter((9 << 32) - 3)
    plant(ws, range(1, 64))
    check_markov("wrap", markov_call(lib, base, left, right, anchor, ws), base, left, right,
                 anchor)
    # top-K on the same memory in the same period, then the one-launch head with tags that the
    # planted words carry: top-K's untagged use makes the head zero-fill the memory first
    lib.sv_set_call_counter((9 << 32) + 1000)
    plant(ws, range(1000, 1000 + 2 * K + 2))
    dev = torch.device("cuda:0")
    tt = torch.empty(B, K, dtype=torch.int32, device=dev)
    st = lib.sv_markov_topk(to_dev(base).data_ptr(), sv.SV_DTYPE_BF16, B, K, V,
                            to_dev(left).data_ptr(), to_dev(right).data_ptr(), R, 16,
                            to_dev(anchor).data_ptr(), tt.data_ptr(), None, None, ws.data_ptr(),
                            ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, sv.sv_last_error()
    check_markov("after top-K", markov_call(lib, base, left, right, anchor, ws), base, left,
                 right, anchor)
    # the per-position form (B = 130) on the same memory, then the one-launch head again
    lib.sv_set_call_counter((9 << 32) + 2000)
    plant(ws, range(2000, 2000 + 2 * K + 2))
    b2, l2, r2, a2 = markov_inputs(130, 2, V, R, 5301)
    check_markov("per-position", markov_call(lib, b2, l2, r2, a2, ws), b2, l2, r2, a2)
    check_markov("after per-position", markov_call(lib, base, left, right, anchor, ws), base,
                 left, right, anchor)


def test_markov_one_launch_beside_a_long_kernel_on_another_stream():
    """A read kernel of a few milliseconds occupies the device from a second stream while the
    one-launch head is enqueued: the cooperative launch still gives exact tokens (the runtime
    places all of its work-groups at once, or the library falls back to the per-position
    form)."""
    lib = sv.load_library()
    B, K, V, R = 64, 8, workloads.QWEN3_VOCAB, 256
    base, left, right, anchor = markov_inputs(B, K, V, R, 5401)
    ws = torch.zeros(int(lib.sv_markov_workspace_bytes(B, V)), dtype=torch.uint8,
                     device="cuda:0")
    solo = markov_call(lib, base, left, right, anchor, ws)
    torch.cuda.synchronize()
    big = torch.ones(1 << 31, dtype=torch.uint8, device="cuda:0")
    side = torch.cuda.Stream()  # default priority
    partial = torch.empty(4096, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        with torch.cuda.stream(side):
            for _ in range(4):
                assert lib.sv_read_probe(big.data_ptr(), big.numel(), partial.data_ptr(), 4096,
                                         side.cuda_stream) == 0
        tok = markov_call(lib, base, left, right, anchor, ws)
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), solo.cpu().numpy())
    check_markov("beside a long kernel", solo, base, left, right, anchor)
