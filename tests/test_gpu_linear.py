"""GPU parity of linear verification: libspecverify through its C ABI against the
oracle, element by element, on seeded synthetic inputs.

Bar: accept lengths and tokens bit-exact. Greedy: always. Stochastic: a
sequence may differ only if one of its evaluated uniforms lies within 1e-6 of
its threshold in the oracle's arithmetic (an exception); exceptions are
counted over the whole session and must stay below 1e-4 of evaluated draws
(checked by test_zz_exception_rate in test_gpu_zz_summary.py). p_target /
p_draft within 1e-5 relative of the oracle's double values."""
import numpy as np
import pytest

import gen
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _check(w, seqs=None):
    G.say(f"{w.name} {w.mode} B={w.B} k={w.k} V={w.V} dtype={w.dtype} T={w.temperature}")
    g = G.run_linear(w)
    o = G.oracle_linear(w, seqs)
    near, n_eval = G.compare_linear(g, o, w.mode == "stochastic", seqs)
    return g, o, near, n_eval


@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_c1_tiny_many_sequences(mode):
    # 20000 independent sequences of the tiny configuration (fp32, V=1000, k=4)
    w = gen.c1_tiny(0, mode, B=20000)
    g, o, exc, n_eval = _check(w)
    if mode == "stochastic":
        assert n_eval > 50000
        assert exc / n_eval < 1e-4, (exc, n_eval)
        # the acceptance rate is in the expected regime (1 - total variation ~ 0.8)
        assert 0.6 < np.mean(g["accept_len"] >= 1) < 0.95
    else:
        assert exc == 0


@pytest.mark.parametrize("dtype", [gen.DT_F32, gen.DT_BF16, gen.DT_F16])
@pytest.mark.parametrize("V", [12345, 20000, 8192, 8193, 3])
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_tiles_and_ragged_tails(dtype, V, mode):
    # several 16 KiB chunks, a partial last chunk, and (V=12345, 8193, 3 in 2-byte
    # dtypes) rows that do not start on a 16-byte boundary
    w = gen.linear_draft_target(90 + dtype, V, 8, 3, V, dtype, 3.0, 1.0, mode, 0.8, f"ragged{V}")
    _check(w)


@pytest.mark.parametrize("V", [262144, 262145, 524288])
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_long_rows(V, mode):
    # fp32 rows of exactly 1 MiB (a target/draft pair's 256 chunk partials fill a
    # wave's four rounds), one element over (each row of a pair combined on its
    # own), and the longest row the library takes (2 MiB)
    w = gen.linear_draft_target(96, V % 7, 3, 2, V, gen.DT_F32, 3.0, 1.0, mode, 0.8, f"long{V}")
    _check(w)


@pytest.mark.parametrize("B", [16, 1200])
def test_zero_residual_falls_back_to_the_target_row(B):
    # One dominant logit, equal in target and draft; every other draft logit is
    # 0.5 above the target's, so the draft token is rejected when u >= about 0.61.
    # In fp32 every residual term rounds to zero (the dominant probabilities agree
    # to about 1e-10), so the draw falls back to softmax of the target row. The
    # exact residual (the oracle) has all its mass on the dominant token, which the
    # fallback draws too unless u lands in a tail of about 1e-10. B = 16 runs in
    # hold mode, B = 1200 (4800 residual waves) queued.
    k, V = 2, 3000
    rng = np.random.default_rng(5)
    dom = rng.integers(0, V, size=(B, k + 1))
    t = np.zeros((B, k + 1, V))
    d = np.full((B, k, V), 0.5)
    t[np.arange(B)[:, None], np.arange(k + 1)[None, :], dom] = 30.0
    d[np.arange(B)[:, None], np.arange(k)[None, :], dom[:, :k]] = 30.0
    tok = (dom[:, :k] + 1 + rng.integers(0, V - 1, size=(B, k))) % V
    u = np.full((B, k + 1), 0.9, np.float32)
    u[:, k] = rng.random(B).astype(np.float32)
    w = gen.LinearWorkload("zero-residual", "stochastic", 1.0, B, k, V, gen.DT_F32, t.astype(np.float32),
                           d.astype(np.float32), tok.astype(np.int32), u)
    g, o, near, n_eval = _check(w)
    assert np.all(g["accept_len"] == 0)
    np.testing.assert_array_equal(g["out_tokens"][:, 0], dom[:, 0])


def test_tiny_draft_token_probabilities():
    # Every draft token sits about 110 natural units below the maxima of both its
    # rows (T = 1), so p_t and p_d are near 1e-52: zero in fp32, ordinary in fp64.
    # Their ratio is e^(-delta) times the ratio of the normalisers, delta uniform in
    # [-1.5, 1.5], so the acceptance test decides on u. Rounded to fp32 both
    # probabilities would vanish and every test would reject.
    B, k, V = 64, 2, 3000
    rng = np.random.default_rng(11)
    t = rng.normal(0.0, 1.0, size=(B, k + 1, V))
    d = rng.normal(0.0, 1.0, size=(B, k, V))
    tok = rng.integers(0, V, size=(B, k))
    bi, ii = np.arange(B)[:, None], np.arange(k)[None, :]
    t[bi, ii, tok] = -110.0
    d[bi, ii, tok] = -110.0 + rng.uniform(-1.5, 1.5, size=(B, k))
    u = gen.uniforms(gen.key(66, V, 2), B * (k + 1)).reshape(B, k + 1)
    w = gen.LinearWorkload("tiny-p", "stochastic", 1.0, B, k, V, gen.DT_F32, t.astype(np.float32),
                           d.astype(np.float32), tok.astype(np.int32), u)
    g, o, near, n_eval = _check(w)
    assert np.all(o["p_target"] < 1e-45) and np.all(o["p_target"] > 0.0)
    assert 0.2 < np.mean(o["accept_len"] >= 1) < 0.95


def test_grouped_residual_waves_odd_chunks():
    # more than 4096 (sequence, chunk) pairs: each residual wave sums two chunks;
    # V = 20000 bf16 rows have 5 chunks, so every sequence's last wave has one
    w = gen.linear_draft_target(97, 0, 1000, 1, 20000, gen.DT_BF16, 3.0, 1.0, "stochastic", 1.0, "grouped")
    g, o, near, n_eval = _check(w)
    assert 0.1 < np.mean(g["accept_len"] == 0) < 0.9


def test_queued_launch_with_few_sequences():
    # 2 MiB fp32 rows have 512 residual waves per sequence, so 8 sequences are more
    # than the GPU keeps waiting at once: the launch is queued, and its decisions
    # take slots (six rejections from the front, two full acceptances from the back)
    w = gen.linear_draft_target(99, 3, 8, 2, 524288, gen.DT_F32, 3.0, 1.0, "stochastic", 0.8, "queued-few")
    g, o, near, n_eval = _check(w)
    assert np.sum(o["accept_len"] == 2) == 2 and np.sum(o["accept_len"] < 2) == 6


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_c2_draft_target_full_size(seed):
    w = gen.c2_linear(seed)            # B=32, k=4, V=128256, bf16, T=0.7
    _check(w)


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_c3_mtp_full_size(mode):
    w = gen.c3_mtp(0, mode)            # D=256, k=1, V=129280, bf16, T=1
    g, o, near, n_eval = _check(w)


def test_identity_accepts_all_plus_bonus():
    w = gen.c2_linear(5, B=8)
    w.draft = np.ascontiguousarray(w.target[:, :w.k, :])
    w.draft_tokens = gen.gumbel_rows(gen.key(2, 5, 9), w.dtype, w.draft, w.V, w.temperature).reshape(w.B, w.k)
    g, o, near, n_eval = _check(w)
    assert np.all(g["accept_len"] == w.k)
    np.testing.assert_array_equal(g["out_tokens"][:, :w.k], w.draft_tokens)
    np.testing.assert_array_equal(g["p_target"], g["p_draft"])


@pytest.mark.parametrize("k", [0, 1, 8, 31])
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_draft_lengths(k, mode):
    w = gen.linear_draft_target(80, k, 6, k, 3000, gen.DT_BF16, 1.0, 0.3, mode, 1.0, f"k{k}")
    _check(w)


def test_argmax_ties_across_chunks():
    # bf16 rows of V=20000 (a wave's chunk holds 4096 bf16 logits): equal maxima
    # placed on both sides of chunk boundaries and in the tail; the lowest index
    # must win
    B, k, V = 6, 2, 20000
    rng = np.random.default_rng(3)
    x = np.round(rng.normal(0, 1, size=(B, k + 1, V)) * 8) / 8
    spots = [(8191, 8192), (8192, 19999), (0, 16384), (16383, 16384), (5, 6), (19998, 19999),
             (4095, 4096), (12287, 16384), (4096, 19999), (19968, 19999)]
    for b in range(B):
        for r in range(k + 1):
            for s in spots[(b + r) % len(spots)]:
                x[b, r, s] = 20.0
    t = gen.round_to(gen.DT_BF16, x)
    am = np.argmax(gen.decode(gen.DT_BF16, t), axis=2)
    tok = am[:, :k].astype(np.int32)
    tok[::2, 1] = (tok[::2, 1] + 1) % V
    w = gen.LinearWorkload("ties", "greedy", 1.0, B, k, V, gen.DT_BF16, t,
                           np.zeros((B, k, V), np.uint16), tok, np.zeros((B, k + 1), np.float32))
    g, o, _, _ = _check(w)
    np.testing.assert_array_equal(g["out_tokens"][1::2, k], am[1::2, k])


def test_data_errors():
    w = gen.linear_draft_target(70, 0, 5, 2, 5000, gen.DT_F16, 2.0, 0.5, "stochastic", 1.0, "errs")
    w.draft_tokens[0, 1] = w.V                       # token out of range
    w.target[1, 1, 77] = 0x7E00                      # NaN (fp16 bits)
    w.draft[2, 0, :] = 0xFC00                        # -inf row
    w.target[3, 2, 10] = 0x7C00                      # +inf
    g, o, _, _ = _check(w)
    assert list(g["err_flags"]) == [1, 2, 2, 2, 0]
    assert list(g["accept_len"][:4]) == [-1] * 4
    wg = gen.linear_draft_target(70, 0, 5, 2, 5000, gen.DT_F16, 2.0, 0.5, "greedy", 1.0, "errs")
    wg.target[1, 1, :] = 0xFC00                      # no usable entry in a target row
    wg.draft_tokens[2, 0] = -1
    g, o, _, _ = _check(wg)
    assert list(g["err_flags"]) == [0, 2, 1, 0, 0]


@pytest.mark.parametrize("B", [6, 2000])
def test_errors_after_a_drawn_rejection(B):
    # Position 0 rejected for sure (the draft puts all its mass on its token, the
    # target almost none), so the final token is the residual draw, which usually
    # comes last; rows after position 0 hold an unusable value in some sequences.
    # The drawing wave that writes the outputs must still see those error bits
    # (hold mode at B = 6, a queued launch at B = 2000).
    w = gen.linear_draft_target(74, 0, B, 2, 1000, gen.DT_F32, 2.0, 0.5, "stochastic", 1.0, f"errs-after{B}")
    x = w.draft_tokens[:, 0]
    w.draft[np.arange(B), 0, x] = 1e4
    w.target[np.arange(B), 0, x] = -1e4
    w.target[0, 1, 5] = np.nan          # position 1, after the rejection
    w.target[1, 2, 7] = np.inf          # target row k
    w.draft[2, 1, :] = -np.inf          # an unusable draft row after the rejection
    g, o, _, _ = _check(w)
    assert list(g["err_flags"][:4]) == [2, 2, 2, 0]
    assert list(g["accept_len"][:4]) == [-1, -1, -1, 0]
    assert np.all(o["accept_len"][3:] == 0)


@pytest.mark.parametrize("case", ["all_accepted", "all_rejected"])
def test_queued_slots_from_one_end(case):
    # A queued launch (MTP shape, 128 sequences) whose decisions all take slots
    # from the back (every draft accepted) or all from the front (every draft
    # rejected): outputs match the oracle and the workspace is all zeros again,
    # the slot word included.
    import torch
    import acceptance_row_softmax_amd as sv
    w = gen.c3_mtp(41, "stochastic", B=128)
    B = w.B
    if case == "all_accepted":
        w.uniforms[:, 0] = 0.0
    else:
        x = w.draft_tokens[:, 0]
        w.draft[np.arange(B), 0, x] = 0x7800    # bf16 bits of 2^113: all the draft's mass
        w.target[np.arange(B), 0, x] = 0xF800   # -2^113: none of the target's
    G.say(f"queued, {case}: B={B} k={w.k} V={w.V}")
    L = sv.lib()
    need = L.spec_verify_linear_workspace(w.B, w.k, w.V, w.dtype, sv.SV_STOCHASTIC)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    t = G.to_dev(w.target, w.dtype)
    d = G.to_dev(w.draft, w.dtype)
    x = G.to_dev(w.draft_tokens.astype(np.int32))
    u = G.to_dev(w.uniforms.astype(np.float32))
    for _ in range(2):
        r = sv.verify_linear(t, d, x, u, mode="stochastic", temperature=w.temperature, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
    got = {k_: (v.cpu().numpy() if v is not None else None) for k_, v in r.items()}
    o = G.oracle_linear(w)
    G.compare_linear(got, o, True)
    assert np.all(o["accept_len"] == (1 if case == "all_accepted" else 0))


def test_deterministic_and_workspace_reuse():
    w1 = gen.c2_linear(7, B=8)
    w2 = gen.c2_linear(8, B=8)
    a = G.run_linear(w1)
    b = G.run_linear(w2)
    c = G.run_linear(w1)
    for key in a:
        if a[key] is not None:
            np.testing.assert_array_equal(a[key], c[key])
    G.compare_linear(b, G.oracle_linear(w2), True)


def test_workspace_left_zero_and_shared_across_shapes():
    """Every record is cleared by its reader: after each call the workspace is all
    zeros again, so one workspace serves calls of different shapes and modes."""
    import torch
    import acceptance_row_softmax_amd as sv
    G.say("one workspace, several shapes; zero after every call")
    wa = gen.c2_linear(9, B=16)
    wb = gen.linear_draft_target(71, 1, 7, 3, 20000, gen.DT_F16, 2.0, 0.5, "greedy", 1.0, "ws-b")
    wc = gen.linear_draft_target(72, 2, 5, 0, 3000, gen.DT_F32, 2.0, 0.5, "stochastic", 1.3, "ws-c")
    wd = gen.c1_tiny(5, "stochastic", B=4000)   # a queued launch (decision slots)
    L = sv.lib()
    # the generator's dtype codes are the library's
    need = max(L.spec_verify_linear_workspace(w.B, w.k, w.V, w.dtype,
                                              sv.SV_STOCHASTIC if w.mode == "stochastic" else sv.SV_GREEDY)
               for w in (wa, wb, wc, wd))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for w in (wa, wb, wc, wd, wa, wd):
        t = G.to_dev(w.target, w.dtype)
        d = G.to_dev(w.draft, w.dtype) if (w.mode == "stochastic" and w.k > 0) else None
        x = G.to_dev(w.draft_tokens) if w.k > 0 else None
        u = G.to_dev(w.uniforms)
        g = sv.verify_linear(t, d, x, u, mode=w.mode, temperature=w.temperature, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, w.name
        got = {k: (v.cpu().numpy() if v is not None else None) for k, v in g.items()}
        G.compare_linear(got, G.oracle_linear(w), w.mode == "stochastic")
