"""Device-side early exit of cached decode against the oracle ("CLI Reference"
page, "generate": the --early-exit-* options).

Effective depths are integers and must equal the oracle's exactly.  The rule
compares floating-point quantities with a threshold, so thresholds are placed
where no probe value of the oracle's run lies within 5 % of them: the GPU's
fp32 values (about 1e-3 away from the fp64 ones) then take the same decisions.
Hidden states meet the usual bars.  Decode is teacher-forced with seeded tokens.
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

SPECS = {
    "tiny-w4": synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128"),
    "tiny-bf16-stack": synth.ModelSpec("tiny-bf16-stack", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16"),
    # wide enough (K = 512: four 128-wide groups) that five lanes' QKV products are
    # split over K and finished inside the decode attention, also on exiting rows
    "mid-w4": synth.ModelSpec("mid-w4", 256, 512, 8, 64, 1024, 1, 1, 0, "f16", "w4g128"),
}
N_LANES, PLEN, STEPS, L0 = 5, 10, 6, 8


def say(*a):
    print("[gpu-ee]", *a, flush=True)
    sys.stdout.flush()


def bar(L):
    return 1e-2 if L <= 8 else 3e-2


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _setup(name, seed=31):
    spec = SPECS[name]
    w = synth.make_weights(spec, seed)
    m = oracle.OracleModel.from_weights(w)
    prompts = [synth.tokens(seed, 5000 + i, PLEN + i, spec.vocab) for i in range(N_LANES)]
    forced = synth.tokens(seed, 5100, N_LANES * STEPS, spec.vocab).reshape(N_LANES, STEPS)
    reqs = synth.uniform_int(seed, 5200, N_LANES * STEPS, 3, L0 - 2).reshape(N_LANES, STEPS)   # 3..L0
    return spec, w, m, prompts, forced, reqs


def _oracle_run(m, prompts, forced, reqs, ee, record=None, monkeypatch=None):
    """Oracle lanes through STEPS early-exit steps; optionally records probe values."""
    if record is not None:
        rd, lm = oracle.model.relative_delta, oracle.model.logit_margin
        monkeypatch.setattr(oracle.model, "relative_delta", lambda hp, h: record.append(rd(hp, h)) or record[-1])
        monkeypatch.setattr(oracle.model, "logit_margin", lambda lg: record.append(lm(lg)) or record[-1])
    lanes = [oracle.prefill(m, p, L0)[0] for p in prompts]
    H, E = np.zeros((STEPS, len(prompts), m.spec.d_model)), np.zeros((STEPS, len(prompts)), np.int32)
    for t in range(STEPS):
        for i, ln in enumerate(lanes):
            h, _, _, e = oracle.decode_step_ee(m, ln, int(reqs[i, t]), ee, token=int(forced[i, t]))
            H[t, i], E[t, i] = h, e
    if record is not None:
        monkeypatch.undo()
    return H, E


def _gpu_run(w, spec, prompts, forced, reqs, ee_kwargs, plain=False):
    caps = [len(p) + STEPS for p in prompts]
    model = load_model(w, max_lanes=8, max_pos=64, max_L=16, kv_arena_bytes=kv_bytes(spec, [L0] * N_LANES, caps))
    try:
        toks = torch.tensor(np.concatenate(prompts), dtype=torch.int32, device="cuda")
        cu = np.cumsum([0] + [len(p) for p in prompts]).astype(np.int32)
        lanes = np.array([3, 0, 6, 1, 5], np.int32)
        tl.tl_forward(model, cu, toks, seq_L=[L0] * N_LANES, lanes=lanes, max_new_tokens=STEPS)
        out = torch.empty(N_LANES, dtype=torch.int32, device="cuda")
        hs = torch.empty(N_LANES, spec.d_model, dtype=torch.float32, device="cuda")
        H, E, T = np.zeros((STEPS, N_LANES, spec.d_model)), np.zeros((STEPS, N_LANES), np.int32), []
        for t in range(STEPS):
            feed = torch.tensor(forced[:, t], dtype=torch.int32, device="cuda")
            if plain:
                e = tl.tl_decode_step(model, lanes, reqs[:, t], out, in_tokens=feed, out_hidden=hs)
            else:
                e = tl.tl_decode_step_ee(model, lanes, reqs[:, t], out, in_tokens=feed, out_hidden=hs, **ee_kwargs)
            torch.cuda.synchronize()
            H[t], E[t] = hs.cpu().numpy(), e
            T.append(out.cpu().numpy().copy())
        return H, E, np.array(T)
    finally:
        tl.tl_free(model)


def _compare(H, E, Hr, Er):
    assert np.array_equal(E, Er), "effective depths differ:\n%s\n%s" % (E, Er)
    for t in range(STEPS):
        for i in range(N_LANES):
            r = rel_l2(H[t, i], Hr[t, i])
            assert r <= bar(int(E[t, i])), (t, i, r)


def _robust_threshold(values, candidates):
    v = np.asarray(values, dtype=np.float64)
    for c in candidates:
        if v.size and np.min(np.abs(v - c) / max(abs(c), 1e-30)) > 0.05:
            return c
    return None


@pytest.mark.parametrize("name", list(SPECS))
def test_ee_disabled_equals_plain_decode(name):
    spec, w, m, prompts, forced, reqs = _setup(name)
    H0, E0, T0 = _gpu_run(w, spec, prompts, forced, reqs, None, plain=True)
    H1, E1, T1 = _gpu_run(w, spec, prompts, forced, reqs, dict(patience=0))
    assert np.array_equal(E0, E1) and np.array_equal(T0, T1)
    assert np.array_equal(H0, H1), "patience 0 must run exactly the plain decode step"


@pytest.mark.parametrize("name", list(SPECS))
@pytest.mark.parametrize("rule", [dict(patience=1, min_L=2, tau=1e30), dict(patience=2, min_L=3, peek_every=2, tau=1e30),
                                  dict(patience=1, min_L=1, tau=0.0), dict(patience=1, min_L=4, logit_margin=1e-30),
                                  dict(patience=2, min_L=2, logit_margin=1e30)])
def test_ee_fixed_outcome_rules_match_oracle(name, rule):
    """Rules whose every probe is stable (or none is): depths follow from the schedule."""
    spec, w, m, prompts, forced, reqs = _setup(name)
    ee = oracle.EarlyExit(rule["patience"], rule.get("min_L", 2), rule.get("tau", 1e-3), rule.get("peek_every", 1),
                          rule.get("logit_margin", 0.0))
    Hr, Er = _oracle_run(m, prompts, forced, reqs, ee)
    H, E, _ = _gpu_run(w, spec, prompts, forced, reqs, rule)
    say(name, rule, "depths", E.tolist())
    _compare(H, E, Hr, Er)


@pytest.mark.parametrize("name", list(SPECS))
@pytest.mark.parametrize("mode", ["hidden", "margin"])
def test_ee_data_dependent_rule_matches_oracle(name, mode, monkeypatch):
    """The rule decides on the model's values: the threshold sits in a gap of the
    oracle's probe values, and the run must take some exits and skip others."""
    spec, w, m, prompts, forced, reqs = _setup(name)
    # the values the rule sees when nobody exits (a never-stable rule probes every
    # eligible iteration), then candidate thresholds at their quantiles
    never = oracle.EarlyExit(1, 2, 0.0, 1, 0.0) if mode == "hidden" else oracle.EarlyExit(1, 2, 0.0, 1, 1e30)
    vals = []
    _, En = _oracle_run(m, prompts, forced, reqs, never, record=vals, monkeypatch=monkeypatch)
    sv = np.unique(np.asarray(vals, dtype=np.float64))
    cands = [0.5 * (a + b) for a, b in zip(sv[:-1], sv[1:]) if (b - a) > 0.1 * abs(0.5 * (a + b))]
    cands.sort(key=lambda c: abs(np.searchsorted(sv, c) - len(sv) / 2))
    thr = None
    for cand in cands:
        ee = (oracle.EarlyExit(1, 2, float(cand), 1, 0.0) if mode == "hidden"
              else oracle.EarlyExit(1, 2, 0.0, 1, float(cand)))
        rec = []
        Hr, Er = _oracle_run(m, prompts, forced, reqs, ee, record=rec, monkeypatch=monkeypatch)
        # robust, some tokens exit early, and not every token at its first probe
        if _robust_threshold(rec, [float(cand)]) is not None and (Er != En).any() and (Er > 2).any():
            thr = float(cand)
            break
    assert thr is not None, "no robust threshold: %d probe values in [%.3g, %.3g], %d gaps" % (
        len(sv), sv.min(), sv.max(), len(cands))
    rule = dict(patience=1, min_L=2, tau=thr) if mode == "hidden" else dict(patience=1, min_L=2, logit_margin=thr)
    H, E, _ = _gpu_run(w, spec, prompts, forced, reqs, rule)
    say(name, mode, "threshold %.4g" % thr, "depths", E.tolist())
    _compare(H, E, Hr, Er)


def test_ee_rejects_invalid_rule():
    spec, w, m, prompts, forced, reqs = _setup("tiny-w4")
    model = load_model(w, max_lanes=8, max_pos=64, max_L=16,
                       kv_arena_bytes=kv_bytes(spec, [L0] * N_LANES, [PLEN + 8] * N_LANES))
    try:
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        for bad in [dict(patience=-1), dict(patience=1, min_L=0), dict(patience=1, peek_every=0),
                    dict(patience=1, tau=-1.0), dict(patience=1, logit_margin=-1.0)]:
            with pytest.raises(tl.TLError) as ei:
                tl.tl_decode_step_ee(model, [0], [4], out, **bad)
            assert ei.value.status == tl.TL_E_ARG
    finally:
        tl.tl_free(model)
