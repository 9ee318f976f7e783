"""Self-speculative decoding on the device against the oracle ("Dynamic-L
Inference" page, "Self-Speculative Decoding"; "CLI Reference" page, "speculate").

Greedy choices are compared exactly, so the prompts are chosen (by seed, searched
in order) such that every greedy decision the oracle takes, in drafts, verify rows
and plain decoding, has a top-1 / top-2 gap far above the device's logit error;
the search also asks for a round that accepts every draft and one that rejects a
draft it could have kept.  Tokens and per-round acceptance must then equal the
oracle's; the tokens must equal the device's own plain greedy decoding at the
verify depth; and teacher-forced steps after the run check the cache left behind
by the rollbacks.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.harness import ensure_built, kv_bytes, load_model, rel_l2

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    # spec, (L_draft, L_verify, draft_ahead), lanes, tokens, relative gap required
    "tiny-fp32": (synth.SPECS[1], (4, 8, 3), 3, 10, 1e-4),
    "tiny-w4": (synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128"), (6, 8, 3), 3, 10, 5e-3),
    "tiny-bf16-stack": (synth.ModelSpec("tiny-bf16-stack", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16"),
                        (6, 8, 2), 1, 6, 3e-2),
    # the MFMA and split-K paths at a 512-wide INT4 model (8 heads x 64)
    "mid-w4": (synth.ModelSpec("mid-w4", 256, 512, 8, 64, 1024, 1, 1, 0, "f16", "w4g128"), (6, 8, 3), 2, 8, 5e-3),
}
L_PRE = 8


def say(*a):
    print("[gpu-spec]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _dev(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


def _oracle_case(m, spec, prompts, Ld, Lv, k, n_tok, monkeypatch):
    """Oracle speculative run and plain greedy run; the smallest relative gap of
    any greedy decision taken in either."""
    gaps = []
    real = oracle.model.greedy_argmax

    def rec(logits):
        lg = np.asarray(logits, dtype=np.float64)
        rows = lg.reshape(-1, lg.shape[-1])
        for r in rows:
            top = np.sort(r)[-2:]
            gaps.append((top[1] - top[0]) / (np.sqrt(np.mean(r * r)) + 1e-30))
        return real(logits)

    monkeypatch.setattr(oracle.model, "greedy_argmax", rec)
    lanes = [oracle.prefill(m, p, L_PRE)[0] for p in prompts]
    res = [oracle.speculative_decode(m, ln, Ld, Lv, k, n_tok) for ln in lanes]
    plain = []
    for p in prompts:
        ln = oracle.prefill(m, p, L_PRE)[0]
        plain.append([oracle.decode_step(m, ln, Lv)[2] for _ in range(n_tok)])
    monkeypatch.undo()
    return lanes, res, plain, min(gaps)


def _rejects(acc, k, n_tok):
    """Some round kept fewer drafts than it could have (not only the last-round cap)."""
    done = 0
    for a in acc:
        if a < min(k, n_tok - done - 1):
            return True
        done += a + 1
    return False


@pytest.mark.parametrize("name", list(CASES))
def test_speculate_matches_oracle(name, monkeypatch):
    spec, (Ld, Lv, k), n, n_tok, need = CASES[name]
    w = synth.make_weights(spec, 71)
    m = oracle.OracleModel.from_weights(w)
    chosen = None
    for seed in range(60):
        prompts = [synth.tokens(71, 8000 + 100 * seed + i, 6 + 3 * i, spec.vocab) for i in range(n)]
        lanes, res, plain, gap = _oracle_case(m, spec, prompts, Ld, Lv, k, n_tok, monkeypatch)
        accs = [a for _, acc in res for a in acc]
        if gap > need and max(accs) == k and any(_rejects(acc, k, n_tok) for _, acc in res):
            chosen = (seed, prompts, lanes, res, plain)
            break
    assert chosen is not None, "no seed with well-separated greedy choices"
    seed, prompts, o_lanes, res, plain = chosen
    for (toks, _), pl in zip(res, plain):
        assert toks == pl                                  # the oracle's own invariant

    cap = max(len(p) for p in prompts) + n_tok + k + 4
    model = load_model(w, max_lanes=8, max_pos=64, max_L=16, kv_arena_bytes=kv_bytes(spec, [L_PRE] * 2 * n, [cap] * 2 * n))
    try:
        spec_lanes = list(range(n))
        plain_lanes = list(range(n, 2 * n))
        for lanes_ in (spec_lanes, plain_lanes):
            cu = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int32)
            tl.tl_forward(model, cu, _dev(np.concatenate(prompts)), L=L_PRE, lanes=lanes_,
                          max_new_tokens=cap - max(len(p) for p in prompts))
        out = torch.empty(n, n_tok, dtype=torch.int32, device="cuda")
        acc = tl.tl_speculate(model, spec_lanes, Ld, Lv, k, n_tok, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        # the device's plain greedy decoding at the verify depth
        step = torch.empty(n, dtype=torch.int32, device="cuda")
        pl = []
        for _ in range(n_tok):
            tl.tl_decode_step(model, plain_lanes, [Lv] * n, step)
            pl.append(step.cpu().numpy().copy())
        pl = np.array(pl).T
        for i in range(n):
            o_toks, o_acc = res[i]
            g_acc = [int(a) for a in acc[i] if a >= 0]
            say(name, "seed", seed, "lane", i, "accepted per round", g_acc)
            assert got[i].tolist() == o_toks, (i, got[i].tolist(), o_toks)
            assert g_acc == o_acc, (i, g_acc, o_acc)
            assert got[i].tolist() == pl[i].tolist()
        # the cache after the rollbacks: teacher-forced steps against the oracle
        feed = synth.tokens(71, 8900, 2 * n, spec.vocab).reshape(2, n)
        hs = torch.empty(n, spec.d_model, dtype=torch.float32, device="cuda")
        bar = 1e-4 if spec.act_dtype == "f32" else 1e-2
        for t in range(2):
            e = tl.tl_decode_step(model, spec_lanes, [16] * n, step, in_tokens=_dev(feed[t]), out_hidden=hs)
            torch.cuda.synchronize()
            H = hs.cpu().numpy()
            for i in range(n):
                h_o, _, _, L_o = oracle.decode_step(m, o_lanes[i], 16, token=int(feed[t, i]))
                assert e[i] == L_o == Lv
                assert rel_l2(H[i], h_o) <= bar, (t, i, rel_l2(H[i], h_o))
    finally:
        tl.tl_free(model)


@pytest.mark.parametrize("mode", ["h8", "d8"])
def test_speculate_in_coded_cache_modes(mode, monkeypatch):
    """Rollbacks in a coded cache mode (the delta chain included): the fp32 model's
    tokens and per-round acceptance equal the oracle's in the same mode.  A code
    can move by one step between the two (x differs by fp32 rounding), so the
    greedy gaps must exceed 1e-2 of the logits' scale."""
    import copy
    spec, (Ld, Lv, k), n, n_tok, _ = CASES["tiny-fp32"]
    modes = {"h8": tl.TL_KV_H8, "d8": tl.TL_KV_D8}
    w = synth.make_weights(spec, 71)
    m = copy.copy(oracle.OracleModel.from_weights(w))
    m.kv_mode = mode
    chosen = None
    for seed in range(60):
        prompts = [synth.tokens(71, 8000 + 100 * seed + i, 6 + 3 * i, spec.vocab) for i in range(n)]
        lanes, res, plain, gap = _oracle_case(m, spec, prompts, Ld, Lv, k, n_tok, monkeypatch)
        accs = [a for _, acc in res for a in acc]
        if gap > 1e-2 and max(accs) == k and any(_rejects(acc, k, n_tok) for _, acc in res):
            chosen = (seed, prompts, res)
            break
    assert chosen is not None, "no seed with well-separated greedy choices"
    seed, prompts, res = chosen
    cap = max(len(p) for p in prompts) + n_tok + k + 4
    model = load_model(w, max_lanes=8, max_pos=64, max_L=16, kv_arena_bytes=kv_bytes(spec, [L_PRE] * n, [cap] * n),
                       kv_mode=modes[mode])
    try:
        cu = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int32)
        tl.tl_forward(model, cu, _dev(np.concatenate(prompts)), L=L_PRE, lanes=list(range(n)),
                      max_new_tokens=cap - max(len(p) for p in prompts))
        out = torch.empty(n, n_tok, dtype=torch.int32, device="cuda")
        acc = tl.tl_speculate(model, list(range(n)), Ld, Lv, k, n_tok, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for i in range(n):
            say(mode, "seed", seed, "lane", i, "accepted per round", [int(a) for a in acc[i] if a >= 0])
            assert got[i].tolist() == res[i][0]
            assert [int(a) for a in acc[i] if a >= 0] == res[i][1]
    finally:
        tl.tl_free(model)


def test_speculate_errors():
    spec = CASES["tiny-w4"][0]
    w = synth.make_weights(spec, 73)
    prompt = synth.tokens(73, 8500, 8, spec.vocab)
    model = load_model(w, max_lanes=4, max_pos=64, max_L=16, kv_arena_bytes=kv_bytes(spec, [8] * 4, [64] * 4))
    try:
        tl.tl_forward(model, np.array([0, 8], np.int32), _dev(prompt), L=8, lanes=[0], max_new_tokens=10)
        out = torch.empty(1, 16, dtype=torch.int32, device="cuda")

        def status(*a):
            with pytest.raises(tl.TLError) as ei:
                tl.tl_speculate(model, *a)
            return ei.value.status

        assert status([0], 2, 8, 4, 7, out) == tl.TL_E_STATE     # 7 + 4 > 10 free positions
        assert status([0], 2, 8, 65, 1, out) == tl.TL_E_ARG      # draft_ahead above 64
        assert status([0], 0, 8, 2, 2, out) == tl.TL_E_ARG       # depth < 1
        assert status([1], 2, 8, 2, 2, out) == tl.TL_E_STATE     # never prefilled
        assert status([0, 0], 2, 8, 2, 2, out) == tl.TL_E_ARG    # repeated lane
        acc = tl.tl_speculate(model, [0], 2, 8, 4, 6, out)       # exactly fits: 6 + 4 = 10
        torch.cuda.synchronize()
        assert sum(int(a) + 1 for a in acc[0] if a >= 0) == 6
    finally:
        tl.tl_free(model)
