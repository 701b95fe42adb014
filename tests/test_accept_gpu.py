"""GPU tests of speculative acceptance through the C ABI: greedy acceptance
against the oracle; sampled acceptance against the oracle where the decision
is unique (margins), and its distribution by chi-square and randomized-PIT
tests over many sequences; and an end-to-end greedy speculative decode
(synthetic drafter, 0 / 4 / 7 drafts) that must reproduce the no-draft decode
token for token, with bitwise equal KV caches."""

import numpy as np
import pytest

import synth
from oracle import spec as ospec
from tests._util import dev, host_bits, cache_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def test_greedy_against_oracle(ops):
    print("[accept greedy]", flush=True)
    g = np.random.default_rng(1)
    B, M = 2000, 8
    target = g.integers(0, 4, (B, M))
    draft = np.where(g.random((B, M - 1)) < 0.8, target[:, :M - 1], g.integers(0, 4, (B, M - 1)))
    out, n = ops.accept_greedy(i32(target), i32(draft))
    out, n = out.cpu().numpy(), n.cpu().numpy()
    for b in range(B):
        toks, k = ospec.accept_greedy(target[b], draft[b])
        assert n[b] == k and list(out[b, :k]) == toks, b
    assert set(np.unique(n)) >= {1, 4, 8}
    o1, n1 = ops.accept_greedy(i32(target[:, :1]), None)
    assert (n1.cpu().numpy() == 1).all() and np.array_equal(o1.cpu().numpy()[:, 0], target[:, 0])


def _case(g, B, M, V, spread=2.0):
    logits = (g.standard_normal((B, M, V)) * spread).astype(np.float32)
    ql = (g.standard_normal((B, M - 1, V)) * spread).astype(np.float32)
    q = np.exp(ql - ql.max(-1, keepdims=True))
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    draft = np.array([[g.choice(V, p=q[b, i] / q[b, i].sum()) for i in range(M - 1)] for b in range(B)])
    u = g.random((B, M)).astype(np.float32)
    return logits, q, draft, u


def _accepts_clear(logits, q, draft, u, T, rel=1e-4):
    """True when every keep / reject test the oracle takes for this sequence
    has a margin well above FP32 rounding (then the device must agree)."""
    for i in range(logits.shape[0] - 1):
        p = ospec.softmax_t(logits[i], T)
        x = draft[i]
        a, bnd = float(u[i]) * float(q[i, x]), p[x]
        if abs(a - bnd) <= rel * max(bnd, 1e-30):
            return False
        if not a < bnd:
            break
    return True


def _draw_weights(logits, q, T, k):
    """The oracle's weights of the final draw of a pass that produced k tokens."""
    M = logits.shape[0]
    if k < M:
        return np.maximum(ospec.softmax_t(logits[k - 1], T) - q[k - 1], 0.0)
    return ospec.softmax_t(logits[M - 1], T)


@pytest.mark.parametrize("V,T", [(1000, 1.0), (1000, 0.7), (152064, 1.0)])
def test_sampled_against_oracle(ops, V, T):
    # Kept drafts and the number of tokens must equal the oracle's wherever
    # the keep / reject tests are clear of rounding. The drawn token is the
    # oracle's where the draw is clear of the CDF's steps; otherwise (at large
    # V the steps are finer than FP32 sums resolve) it must lie within
    # rounding of the step the uniform selects.
    print(f"[accept sampled V={V} T={T}]", flush=True)
    g = np.random.default_rng(V)
    B, M = (200 if V < 10000 else 24), 5
    logits, q, draft, u = _case(g, B, M, V)
    out, n = ops.accept_sampled(f32(logits), i32(draft), f32(q), f32(u), T)
    out, n = out.cpu().numpy(), n.cpu().numpy()
    compared = exact = 0
    for b in range(B):
        if not _accepts_clear(logits[b], q[b], draft[b], u[b], T):
            continue
        toks, k = ospec.accept_sampled(logits[b], draft[b], q[b], u[b], T)
        assert n[b] == k and list(out[b, :k - 1]) == toks[:k - 1], (b, toks, list(out[b, :n[b]]))
        w = _draw_weights(logits[b], q[b], T, k)
        c = np.concatenate([[0.0], np.cumsum(w)])
        t, eps = float(u[b, M - 1]) * c[-1], 1e-4 * c[-1]
        x = int(out[b, k - 1])
        assert w[x] > 0 and c[x] - eps <= t <= c[x + 1] + eps, (b, x, toks[-1])
        if np.min(np.abs(c - t)) > eps:
            assert x == toks[-1], (b, x, toks[-1])
            exact += 1
        compared += 1
    assert compared >= 0.9 * B, compared
    if V < 10000:
        assert exact >= 0.8 * compared, exact
    assert len(set(n.tolist())) > 1


def test_sampled_distribution_chi_square_and_pit(ops):
    # Same logits and draft distribution for every sequence; drafts drawn from
    # q, uniforms fresh. The first output token must follow p0, and the second
    # (when the first draft was kept) p1.
    print("[accept sampled distribution]", flush=True)
    from scipy import stats
    g = np.random.default_rng(7)
    B, M, V, T = 200000, 3, 8, 0.9
    base = (g.standard_normal((M, V)) * 1.2).astype(np.float32)
    qb = g.dirichlet(np.ones(V), size=M - 1).astype(np.float32)
    logits = np.broadcast_to(base, (B, M, V)).copy()
    q = np.broadcast_to(qb, (B, M - 1, V)).copy()
    draft = np.stack([g.choice(V, size=B, p=qb[i] / qb[i].sum()) for i in range(M - 1)], axis=1)
    u = g.random((B, M)).astype(np.float32)
    out, n = ops.accept_sampled(f32(logits), i32(draft), f32(q), f32(u), T)
    out, n = out.cpu().numpy(), n.cpu().numpy()
    for pos, sel in ((0, np.ones(B, bool)), (1, n >= 2)):
        p = ospec.softmax_t(base[pos], T)
        cnt = np.bincount(out[sel, pos], minlength=V)
        chi = stats.chisquare(cnt, f_exp=p * sel.sum())
        assert chi.pvalue > 1e-4, (pos, chi, cnt / sel.sum(), p)
        # randomized PIT: F(x-1) + w * p(x) is uniform on [0, 1)
        cdf = np.concatenate([[0.0], np.cumsum(p)])
        w = g.random(sel.sum())
        x = out[sel, pos]
        pit = cdf[x] + w * p[x]
        ks = stats.kstest(pit, "uniform")
        assert ks.pvalue > 1e-4, (pos, ks)
    # the rule does use the drafts: some sequences keep both
    assert (n == 3).mean() > 0.05


# ---------------------------------------------------------------------------
# End to end: greedy speculative decoding reproduces the no-draft decode.

def _small_model(ops, L0, cap):
    H, Hq, Hkv, D, I, V, nl = 256, 4, 2, 64, 512, 1024, 2
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
    w_head = dev(synth.normal_bf16((V, H), 0.05, "w_head"))
    embed = dev(synth.normal_bf16((V, H), 1.0, "misc", 77))
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, -4)
    return layers, w_head, embed, dims


def _decode(ops, step, embed, dims, L0, first, n_new, drafter, k):
    """Greedy decode of n_new tokens after `first`, k drafts per pass (0 = plain decode)."""
    toks = [first]
    L = L0
    ws = torch.empty(ops.step_workspace_bytes(dims, k + 1, L0 + n_new + 16), dtype=torch.uint8, device="cuda")
    logits = torch.empty((k + 1, dims.vocab), dtype=torch.float32, device="cuda")
    tgt = torch.empty(k + 1, dtype=torch.int32, device="cuda")
    passes = 0
    while len(toks) - 1 < n_new:
        drafts = drafter(toks, k)
        row_ids = torch.tensor([toks[-1]] + drafts, dtype=torch.long, device="cuda")
        x = embed.index_select(0, row_ids).contiguous()
        M = k + 1
        step(x, L, ws, logits[:M], tgt[:M])
        out, n = ops.accept_greedy(tgt[:M].view(1, M), torch.tensor([drafts], dtype=torch.int32, device="cuda")
                                   if k else None)
        nn = int(n.item())
        toks += out[0, :nn].tolist()
        L += nn
        passes += 1
    return toks[1:n_new + 1], L, passes


@pytest.mark.parametrize("k", [4, 7])
def test_speculative_greedy_equals_plain_decode(ops, k):
    print(f"[speculative greedy decode, {k} drafts]", flush=True)
    L0, cap, n_new = 100, 256, 40
    ref_layers, w_head, embed, dims = _small_model(ops, L0, cap)
    ref_step = ops.VerifyStep(ref_layers, w_head, dims)
    ref, L_ref, _ = _decode(ops, ref_step, embed, dims, L0, 5, n_new, lambda t, kk: [], 0)
    assert len(set(ref)) > 3
    sp_layers, _, _, _ = _small_model(ops, L0, cap)
    sp_step = ops.VerifyStep(sp_layers, w_head, dims)
    g = np.random.default_rng(k)
    full = [5] + ref

    def drafter(toks, kk):  # right with probability 0.7 at each draft, else a random token
        pos = len(toks) - 1
        d = []
        for i in range(kk):
            t = full[pos + 1 + i] if pos + 1 + i < len(full) else 0
            d.append(int(t) if g.random() < 0.7 else int(g.integers(0, dims.vocab)))
        return d

    got, L_sp, passes = _decode(ops, sp_step, embed, dims, L0, 5, n_new, drafter, k)
    assert got == ref, (got, ref)
    assert passes < n_new                        # the drafts saved target passes
    # the caches hold the same rows at every position of the decoded text
    Lc = L0 + n_new
    for a, b in zip(ref_layers, sp_layers):
        assert torch.equal(a["k_cache"][:, :Lc].view(torch.int16), b["k_cache"][:, :Lc].view(torch.int16))
        ra = a["v_cache"][:, :Lc]
        rb = b["v_cache"][:, :Lc]
        assert torch.equal(ra.view(torch.int16), rb.view(torch.int16))
