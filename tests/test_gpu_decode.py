"""GPU parity of gdr_decode_step against the oracle's single-step recurrence.

Tolerance: max|Δ|/rms(ref) <= 1e-4 with fp32 activations, <= 2e-2 with bf16
activations (fp32 state and decay in both), on o and on the updated state."""
import numpy as np
import pytest

import gdr_synth as gs
import oracle
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu


def _dev(tok, act):
    import torch
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    return {n: torch.from_numpy(np.ascontiguousarray(a)).to(
        torch.float32 if n == "log_alpha" else dt).cuda() for n, a in tok.items()}


CASES = [
    # N, H, dk, dv, act, alpha, b, w
    (4, 3, 128, 128, "bf16", "channel", "channel", "channel"),
    (4, 3, 128, 128, "f32", "channel", "channel", "channel"),
    (2, 5, 64, 64, "bf16", "scalar", "scalar", "scalar"),
    (3, 2, 16, 16, "f32", "scalar", "scalar", "scalar"),
    (3, 2, 32, 128, "f32", "channel", "scalar", "channel"),
    (3, 2, 128, 16, "bf16", "channel", "channel", "scalar"),
    (1, 1, 64, 32, "f32", "channel", "channel", "channel"),
    # more heads, and a single one
    (16, 32, 128, 128, "bf16", "channel", "channel", "channel"),
    (10, 20, 128, 128, "bf16", "channel", "channel", "channel"),
    (5, 20, 128, 128, "f32", "channel", "scalar", "channel"),
    (1, 1, 128, 128, "f32", "scalar", "channel", "scalar"),
    (10, 20, 64, 64, "bf16", "channel", "channel", "channel"),
    (5, 20, 64, 64, "f32", "scalar", "scalar", "channel"),
]


@pytest.mark.parametrize("N,H,dk,dv,act,am,bm,wm", CASES)
def test_decode_steps_match_oracle(N, H, dk, dv, act, am, bm, wm):
    import torch
    import gated_delta_rule_24_amd as gdr
    print(f"decode case N={N} H={H} dk={dk} dv={dv} {act} {am}/{bm}/{wm}", flush=True)
    S = gs.decode_state(N, H, dk, dv, seed=1)
    Sd = torch.from_numpy(S).cuda()
    Sref = S.astype(np.float64)
    tol = 1e-4 if act == "f32" else 2e-2
    for step in range(5):
        tok = gs.decode_token(N, H, dk, dv, step, seed=1, act=act, alpha_mode=am, b_mode=bm,
                              w_mode=wm)
        d = _dev(tok, act)
        o = gdr.decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], Sd)
        o_ref, Sref = oracle.decode(tok["q"], tok["k"], tok["v"], tok["log_alpha"], tok["b"],
                                    tok["w"], Sref)
        torch.cuda.synchronize()
        assert rel_err(o.cpu().numpy(), o_ref) <= tol
        assert rel_err(Sd.cpu().numpy(), Sref) <= tol


def test_decode_bf16_output_is_rounded_fp32_output():
    import torch
    import gated_delta_rule_24_amd as gdr
    N, H, d = 8, 4, 128
    S = gs.decode_state(N, H, d, d, seed=2)
    tok = _dev(gs.decode_token(N, H, d, d, 0, seed=2), "bf16")
    S1 = torch.from_numpy(S).cuda()
    S2 = S1.clone()
    o32 = gdr.decode_step(tok["q"], tok["k"], tok["v"], tok["log_alpha"], tok["b"], tok["w"], S1)
    o16 = gdr.decode_step(tok["q"], tok["k"], tok["v"], tok["log_alpha"], tok["b"], tok["w"], S2,
                          out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(S1, S2)


def test_decode_full_workload_sampled():
    """The decode workload: 256 sequences x 32 heads, d=128, fp32 state updated
    in place over its 128 steps.  Every head is checked after step 1, and a
    sample of 64 heads is followed over all 128 steps (output of every step,
    state at the end)."""
    import torch
    import gated_delta_rule_24_amd as gdr
    N, H = gs.DECODE["N"], gs.DECODE["H"]
    d = gs.DECODE["dk"]
    S = gs.decode_state(N, H, d, d, seed=0)
    Sd = torch.from_numpy(S).cuda()
    rng = np.random.default_rng(5)
    pick = rng.choice(N * H, size=64, replace=False)
    Sref = S.reshape(N * H, d, d)[pick].astype(np.float64)
    for step in range(gs.DECODE["steps"]):
        tok = gs.decode_token(N, H, d, d, step, seed=0)
        dv = _dev(tok, "bf16")
        o = gdr.decode_step(dv["q"], dv["k"], dv["v"], dv["log_alpha"], dv["b"], dv["w"], Sd)
        flat = {n: a.reshape((N * H,) + a.shape[2:]) for n, a in tok.items()}
        if step == 0:
            o_all, S_all = oracle.decode(flat["q"], flat["k"], flat["v"], flat["log_alpha"],
                                         flat["b"], flat["w"], S.reshape(N * H, d, d))
            torch.cuda.synchronize()
            assert rel_err(o.cpu().numpy().reshape(N * H, d), o_all) <= 2e-2
            assert rel_err(Sd.cpu().numpy().reshape(N * H, d, d), S_all) <= 2e-2
        o_ref, Sref = oracle.decode(*(flat[n][pick] for n in ("q", "k", "v", "log_alpha", "b", "w")),
                                    Sref)
        torch.cuda.synchronize()
        assert rel_err(o.cpu().numpy().reshape(N * H, d)[pick], o_ref) <= 2e-2
    assert rel_err(Sd.cpu().numpy().reshape(N * H, d, d)[pick], Sref) <= 2e-2


def test_decode_steps_replay_from_a_graph():
    """A run of decode steps captured into a graph (how a serving loop avoids
    a launch per step at small batch) replays to the eager results, bit for
    bit, on several replays with eager work between them."""
    import torch
    import gated_delta_rule_24_amd as gdr
    N, H, D, K = 2, 8, 128, 6
    print(f"decode graph N={N} H={H} d={D} steps={K}", flush=True)
    S_init = torch.from_numpy(gs.decode_state(N, H, D, D, seed=3)).cuda()
    toks = []
    for st in range(K):
        t = gs.decode_token(N, H, D, D, st, seed=3)
        toks.append({n: torch.from_numpy(a).to(torch.float32 if n == "log_alpha"
                                               else torch.bfloat16).cuda() for n, a in t.items()})
    outs = [torch.empty((N, H, D), dtype=torch.float32, device="cuda") for _ in range(K)]
    S = S_init.clone()

    def run():
        for i, t in enumerate(toks):
            gdr.gdr_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"], S, outs[i],
                                N, H, D, D, 0)
    run()
    torch.cuda.synchronize()
    eager_o = [o.clone() for o in outs]
    eager_S = S.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        S.copy_(S_init)
        for o in outs:
            o.zero_()
        x = torch.randn(1 << 20, device="cuda")
        x.mul_(2.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, eager_S), rep
        for i in range(K):
            assert torch.equal(outs[i], eager_o[i]), (rep, i)
