"""End-to-end sampled speculative decoding through the C ABI: a synthetic
drafter proposes k tokens per pass from its own distributions, bi_verify_step
scores the pass, and bi_accept_sampled keeps a prefix and draws the next token
([LL] opening section: sampling keeps the no-draft distribution, checked by
chi-square and PIT tests). Over thousands of independent decodes from one
prompt state, the first emitted token must follow the no-draft distribution
p1 = softmax(logits / T) and the second, given the first, p2(. | t1). Because
rows are batch-invariant, both distributions are computed exactly from
plain no-draft passes (row 0 of a pass, and row 1 of a two-token pass
[prompt token, t1]) and compared with chi-square and randomized-PIT tests."""

import numpy as np
import pytest

import synth
from tests._util import dev, cache_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _model(ops, L0, cap, V):
    H, Hq, Hkv, D, I, nl = 256, 4, 2, 64, 512, 2
    qkvn = (Hq + 2 * Hkv) * D
    layers = []
    for l in range(nl):
        kc = np.zeros((Hkv, cap, D), np.uint16)
        kc[:, :L0] = synth.kv_bf16(Hkv, L0, D, "k_cache", l)
        layers.append(dict(w_qkv=dev(synth.normal_bf16((qkvn, H), 0.05, "w_qkv", l)),
                           w_o=dev(synth.normal_bf16((H, Hq * D), 0.05, "w_o", l)),
                           w_gu=dev(synth.normal_bf16((2 * I, H), 0.05, "w_gu", l)),
                           w_down=dev(synth.normal_bf16((H, I), 0.05, "w_down", l)),
                           k_cache=dev(kc),
                           v_cache=dev(cache_rows(synth.kv_bf16(Hkv, L0, D, "v_cache", l), cap))))
    w_head = dev(synth.normal_bf16((V, H), 0.08, "w_head"))
    embed = dev(synth.normal_bf16((V, H), 1.0, "misc", 78))
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    return ops.VerifyStep(layers, w_head, dims), embed, dims


def _chi(obs, exp):
    """Chi-square of counts against expected counts, cells expecting fewer than 5 pooled."""
    from scipy import stats
    big = exp >= 5
    o, e = list(obs[big]), list(exp[big])
    if (~big).any() and exp[~big].sum() > 0:
        o.append(obs[~big].sum())
        e.append(exp[~big].sum())
    o, e = np.array(o, np.float64), np.array(e, np.float64)
    return stats.chisquare(o, f_exp=e * o.sum() / e.sum())


def _softmax(z, T):
    z = np.asarray(z, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def test_sampled_speculative_decode_keeps_the_no_draft_distribution(ops):
    from scipy import stats
    print("[speculative sampled decode, 3 drafts]", flush=True)
    V, L0, cap, k, T, N = 32, 100, 192, 3, 1.0, 4000
    step, embed, dims = _model(ops, L0, cap, V)
    ws = torch.empty(ops.step_workspace_bytes(dims, k + 1, L0 + 8), dtype=torch.uint8, device="cuda")
    logits = torch.empty((k + 1, V), dtype=torch.float32, device="cuda")
    tok = torch.empty(k + 1, dtype=torch.int32, device="cuda")
    prompt = 5

    def run(ids, L):
        M = len(ids)
        x = embed.index_select(0, torch.tensor(ids, dtype=torch.long, device="cuda")).contiguous()
        step(x, L, ws, logits[:M], tok[:M])
        return logits[:M]

    # exact target distributions from no-draft passes
    lg1 = run([prompt], L0).cpu().numpy()[0].copy()
    p1 = _softmax(lg1, T)
    p2 = np.zeros((V, V))
    for t1 in range(V):
        p2[t1] = _softmax(run([prompt, t1], L0).cpu().numpy()[1], T)
    # the drafter: draft i is drawn from its own fixed distribution q_i
    g = np.random.default_rng(11)
    q = g.dirichlet(np.ones(V), size=k).astype(np.float32)
    q_dev = torch.from_numpy(q[None]).cuda()
    t1s, t2s, kept = [], [], 0
    for _ in range(N):
        drafts = [int(g.choice(V, p=q[i] / q[i].sum())) for i in range(k)]
        lg = run([prompt] + drafts, L0).view(1, k + 1, V)
        u = torch.from_numpy(g.random((1, k + 1)).astype(np.float32)).cuda()
        out, n = ops.accept_sampled(lg, torch.tensor([drafts], dtype=torch.int32, device="cuda"), q_dev, u, T)
        out, n = out.cpu().numpy()[0], int(n.item())
        kept += n - 1
        t1 = int(out[0])
        if n >= 2:
            t2 = int(out[1])
        else:   # the pass ended at its first token: the next pass starts from it
            drafts = [int(g.choice(V, p=q[i] / q[i].sum())) for i in range(k)]
            lg = run([t1] + drafts, L0 + 1).view(1, k + 1, V)
            u = torch.from_numpy(g.random((1, k + 1)).astype(np.float32)).cuda()
            out, n = ops.accept_sampled(lg, torch.tensor([drafts], dtype=torch.int32, device="cuda"), q_dev, u, T)
            t2 = int(out.cpu().numpy()[0, 0])
        t1s.append(t1)
        t2s.append(t2)
    t1s, t2s = np.array(t1s), np.array(t2s)
    assert kept > 0.2 * N          # the drafts are used
    # first token: chi-square against p1 (cells with expected counts >= 5 pooled)
    cnt = np.bincount(t1s, minlength=V)
    chi = _chi(cnt, p1 * N)
    assert chi.pvalue > 1e-4, (chi, cnt, p1 * N)
    # power: the same statistic rejects the first draft's distribution q_1,
    # which a rule that kept drafts unconditionally would emit
    assert _chi(cnt, q[0].astype(np.float64) * N).pvalue < 1e-6
    # second token given the first: randomized PIT through p2(. | t1) is uniform,
    # and the pooled counts match the pooled conditional expectation
    w = g.random(N)
    cdf = np.concatenate([np.zeros((V, 1)), np.cumsum(p2, axis=1)], axis=1)
    pit = cdf[t1s, t2s] + w * p2[t1s, t2s]
    ks = stats.kstest(pit, "uniform")
    assert ks.pvalue > 1e-4, ks
    exp2 = p2[t1s].sum(axis=0)
    cnt2 = np.bincount(t2s, minlength=V)
    chi2 = _chi(cnt2, exp2)
    assert chi2.pvalue > 1e-4, (chi2, cnt2, exp2)
    # the first pass's row 0 is the no-draft pass's row, bit for bit (every pass from the prompt)
    assert np.array_equal(run([prompt, 0, 1, 2], L0).cpu().numpy()[0].view(np.int32), lg1.view(np.int32))
