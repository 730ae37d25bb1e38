"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream, allocates
nothing and never synchronises, so a sequence of calls can be captured once
and replayed. The graph here holds a causal GQA prefill, its backward, a
packed-document prefill, a split-K decode, a paged decode and the
no-allocation split-K decode. It is replayed
three times with eager work and synchronisations in between (the outputs are
overwritten with NaN before each replay), and every replay must reproduce
the eager results bit for bit: the kernels are deterministic and none reads
memory that it did not write first.
"""

import math

import numpy as np
import pytest
import torch

import exact_io_aware_06_amd as mi

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make_inputs():
    g = torch.Generator().manual_seed(77)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)
    B, H, Hkv, N, d = 1, 4, 2, 300, 128
    x = {"q": r(B, H, N, d), "k": r(B, Hkv, N, d), "v": r(B, Hkv, N, d), "do": r(B, H, N, d)}
    # packed documents of 70, 1 and 129 tokens
    x["qp"], x["kp"], x["vp"] = r(H, 200, d), r(Hkv, 200, d), r(Hkv, 200, d)
    x["cu"] = torch.tensor([0, 70, 71, 200], dtype=torch.int32, device=DEV)
    # decode: 3 sequences over a 1000-key cache, and the same keys in 16-key pages
    x["qd"], x["kc"], x["vc"] = r(3, H, d), r(3, Hkv, 1000, d), r(3, Hkv, 1000, d)
    lens = [1000, 37, 512]
    x["lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ps = 16
    npp = [-(-n // ps) for n in lens]
    perm = np.random.default_rng(5).permutation(sum(npp))
    table = np.zeros((3, max(npp)), dtype=np.int32)
    kpg = torch.zeros(sum(npp), Hkv, ps, d, dtype=torch.bfloat16, device=DEV)
    vpg = torch.zeros_like(kpg)
    nxt = 0
    for b in range(3):
        for j in range(npp[b]):
            pg = int(perm[nxt])
            nxt += 1
            table[b, j] = pg
            n = min(ps, lens[b] - j * ps)
            kpg[pg, :, :n] = x["kc"][b, :, j * ps:j * ps + n]
            vpg[pg, :, :n] = x["vc"][b, :, j * ps:j * ps + n]
    x["kpg"], x["vpg"], x["table"] = kpg, vpg, torch.from_numpy(table).to(DEV)
    return x


def run_all(x):
    s = 1 / math.sqrt(128)
    o, lse = mi.attn_fwd(x["q"], x["k"], x["v"], scale=s, causal=1)
    dq, dk, dv = mi.attn_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], scale=s, causal=1)
    op, lp = mi.attn_fwd_varlen(x["qp"], x["kp"], x["vp"], x["cu"], x["cu"], 129, scale=s,
                                causal=True)
    od, ld = mi.attn_decode(x["qd"], x["kc"], x["vc"], scale=s, num_splits=7)
    og, lg = mi.attn_decode_paged(x["qd"], x["kpg"], x["vpg"], x["table"], x["lens"], scale=s,
                                  num_splits=5)
    # the same keys in the contiguous cache with per-sequence lengths (plan, pieces, merge)
    ov, lv = mi.attn_decode_varlen(x["qd"], x["kc"], x["vc"], x["lens"], scale=s, num_splits=5)
    # the no-allocation decode (its partials in the library's own scratch)
    on = torch.empty_like(x["qd"])
    ln = torch.empty(x["qd"].shape[:2], dtype=torch.float32, device=DEV)
    mi.attn_decode_splitk_noalloc(x["qd"], x["kc"], x["vc"], on, ln, scale=s, num_splits=7)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "op": op, "lp": lp, "od": od,
            "ld": ld, "og": og, "lg": lg, "ov": ov, "lv": lv, "on": on, "ln": ln}


def test_graph_replays_match_eager():
    x = make_inputs()
    eager = run_all(x)
    torch.cuda.synchronize()
    eager = {k: t.clone() for k, t in eager.items()}

    # warm up on a side stream, as capture requires, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run_all(x)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        # eager library work between replays, on the current stream; the
        # no-allocation decode overwrites the scratch with another shape
        mi.attn_fwd(x["q"], x["k"], x["v"], scale=0.05, causal=0)
        qx, kx = x["qd"][:2].contiguous(), x["kc"][:2, :, :600].contiguous()
        mi.attn_decode_splitk_noalloc(qx, kx, kx, torch.empty_like(qx),
                                      torch.empty(qx.shape[:2], device=DEV), scale=0.1,
                                      num_splits=3 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, ref in eager.items():
            assert torch.equal(outs[name], ref), f"replay {rep}: {name} differs from the eager call"
    # the no-allocation decode equals the decode with a workspace, and the paged cache the
    # contiguous one holding the same keys
    assert torch.equal(eager["on"], eager["od"]) and torch.equal(eager["ln"], eager["ld"])
    assert torch.equal(eager["og"], eager["ov"]) and torch.equal(eager["lg"], eager["lv"])
