"""Graph capture of every entry-point family.

The library allocates nothing, issues no memset and never synchronises (the
L2 norm's workspace is cleared by its finalize kernel), so a sequence of calls
can be captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed. The
test captures the full-vocabulary logprob (groups 1 and 2), the nucleus path
with its support records, the backward, the L2 norm, the LM-head linear and the
fused linear + logprob; it replays the graph several times with other eager
work, output poisoning and synchronisations between the replays, and checks
every replay's bytes against the eager calls.
"""
import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def test_graph_replays_match_eager():
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77)
    say("case: graph capture, 96 x 10240 logits, 300 x 256 x 3000 linear, 300001-value norm")
    n, vp, vr = 96, 10240, 10000
    x = rng.normal(0.0, 2.5, (n, vp)).astype(np.float32)
    bits = datagen.f32_to_bf16_bits(x)
    bits[:, vr:] = 0xFF80
    lg = torch.from_numpy(bits.view(np.int16)).to(dev)
    T = torch.from_numpy(rng.choice(np.array([0.7, 1.0, 1.3, 0.0], np.float32), n)).to(dev)
    P = torch.from_numpy(rng.choice(np.array([0.9, 0.99, 1.0], np.float32), n)).to(dev)
    K = torch.from_numpy(rng.choice(np.array([-1, 50, 9000], np.int32), n)).to(dev)
    tg = torch.from_numpy(rng.integers(0, vr, n).astype(np.int64)).to(dev)
    gr = torch.from_numpy(rng.normal(0, 1, n).astype(np.float32)).to(dev)
    gp = torch.from_numpy(rng.normal(0, 1, n).astype(np.float32)).to(dev)
    xv = torch.from_numpy(datagen.grad_values(5, 300_001)).to(dev)
    hb, wb = datagen.linear_exact_inputs(6, 300, 256, 3000)
    hh = torch.from_numpy(hb.view(np.int16)).to(dev)
    ww = torch.from_numpy(wb.view(np.int16)).to(dev)
    vpl = 3072
    Tl = torch.full((300,), 0.7, dtype=torch.float32, device=dev)
    tgl = torch.from_numpy(rng.integers(0, 3000, 300).astype(np.int64)).to(dev)

    def f32(m):
        return torch.empty(m, dtype=torch.float32, device=dev)

    full_out, full_lse, full2_out = f32(n), f32(n), f32(n)
    pol, ref, lse_n = f32(n), f32(n), f32(n)
    state = torch.empty((n, 4), dtype=torch.int32, device=dev)
    grad = torch.empty((n, vp), dtype=torch.int16, device=dev)
    sumsq = torch.empty(1, dtype=torch.float64, device=dev)
    norm = f32(1)
    ws_norm = torch.zeros(rlk.NORM_BIN_WORDS, dtype=torch.int64, device=dev)
    lin_logits = torch.empty((300, vpl), dtype=torch.int16, device=dev)
    lin_out, lin_lse = f32(300), f32(300)
    lin_ws = torch.empty(rlk.linear_logp_workspace_bytes(300, vpl, 3000), dtype=torch.uint8, device=dev)
    ws_full2 = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    ws_nuc = torch.empty(1 << 20, dtype=torch.uint8, device=dev)

    def run():
        rlk.logp_full(lg, T, tg, vocab_real=vr, return_lse=True, out=full_out, lse_out=full_lse)
        rlk.logp_full(lg, T, tg, vocab_real=vr, groups=2, out=full2_out, workspace=ws_full2)
        rlk.logp_nucleus(lg, T, P, K, tg, vocab_real=vr, return_state=True, policy_out=pol, ref_out=ref,
                         lse_out=lse_n, state_out=state, workspace=ws_nuc)
        rlk.logp_backward(lg, T, tg, vocab_real=vr, ref_logp=ref, lse=lse_n, grad_ref=gr, policy_logp=pol,
                          support_state=state, grad_policy=gp, out=grad)
        rlk.l2norm(xv, workspace=ws_norm, sumsq_out=sumsq, norm_out=norm)
        rlk.linear(hh, ww, vocab_padded=vpl, out=lin_logits)
        rlk.linear_logp(hh, ww, Tl, tgl, vocab_padded=vpl, return_lse=True, out=lin_out, lse_out=lin_lse,
                        workspace=lin_ws)

    outs = [full_out, full_lse, full2_out, pol, ref, lse_n, state, grad, sumsq, norm, lin_logits, lin_out, lin_lse]
    run()
    torch.cuda.synchronize()
    want = [o.cpu().numpy().tobytes() for o in outs]
    # groups never change the logprob
    assert np.array_equal(full_out.cpu().numpy().view(np.uint32), full2_out.cpu().numpy().view(np.uint32))

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    for rep in range(4):
        for o in outs:
            if o.dtype in (torch.float32, torch.float64):
                o.fill_(float("nan"))
            else:
                o.fill_(-7)
        junk = torch.randn(4096, device=dev)
        (junk * junk).sum().item()          # other eager work and a synchronisation between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy().tobytes() for o in outs]
        for i, (a, b) in enumerate(zip(got, want)):
            assert a == b, f"replay {rep}: output {i} differs from the eager call"
        say(f"replay {rep}: all {len(outs)} outputs equal the eager bytes")
    # the norm's workspace is left zero after every replay
    assert int(torch.count_nonzero(ws_norm).item()) == 0
