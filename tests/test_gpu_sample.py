"""GPU parity of ev_node_sample (the per-node draw of sampled verification at temperature > 0)
against the CPU oracle, the law of the GPU draws, and the sampled step (draws + acceptance)."""
import numpy as np
import pytest

import oracle
from draft_tree_verification_amd import synth
from draft_tree_verification_amd.synth import BF16, F32

from . import gpu_util as gu
from .pins import _chi2_ok, _softmax

pytestmark = pytest.mark.gpu


def _gpu_sample(raw, T, seed, offset, vocab=None):
    import torch
    from draft_tree_verification_amd import ev
    tok, _ = ev.node_sample(gu.to_dev(raw), temperature=T, seed=seed, offset=offset, vocab=vocab)
    torch.cuda.synchronize()
    return tok.cpu().numpy()


def _check_draws(raw, T, seed, offset, vocab=None, what=""):
    """Tokens equal the oracle's; where they differ, the two tokens' scores must tie to within a
    few ulps (the device log2 may differ from the host's in the last place)."""
    stride = raw.shape[1]
    vocab = vocab or stride
    got = _gpu_sample(raw, T, seed, offset, vocab)
    ref, ref_score = oracle.node_sample(raw, T, seed, offset, vocab=vocab, row_stride=stride)
    bad = np.nonzero(got != ref)[0]
    z = gu.widen(raw)
    for r in bad:
        g = int(got[r])
        assert 0 <= g < vocab, f"{what}: row {r} drew {g} outside the vocabulary"
        s_g = oracle.sample_score(float(z[r, g]), T, seed, offset, int(r), g)
        # each score carries the device log2's error (about 2e-6 absolute at most here)
        tol = 1e-5 + 8 * np.spacing(np.float32(max(1.0, abs(float(ref_score[r])))))
        assert s_g >= float(ref_score[r]) - tol, \
            f"{what}: row {r}: gpu {g} (score {s_g}) vs oracle {ref[r]} (score {ref_score[r]})"
    assert len(bad) <= max(1, len(got) // 1000), f"{what}: {len(bad)} near-tie differences"
    return got


@pytest.mark.parametrize("T", [0.6, 1.0])
def test_workload_c8(T):
    gu.log(f"[case] sample c8 T={T}")
    w = gu.cached_config("c8")
    _check_draws(w.logits, T, seed=1234, offset=7, what=f"c8 T={T}")


def test_workload_c512_rows():
    gu.log("[case] sample c512 first rows")
    w = gu.cached_config("c512")
    _check_draws(np.ascontiguousarray(w.logits[:256]), 1.0, seed=99, offset=3, what="c512")


@pytest.mark.parametrize("R,V,stride,dtype,T", [(3, 151936, 151936, F32, 1.0), (40, 1001, 1008, BF16, 0.05),
                                                (40, 1001, 1008, F32, 10.0), (7, 5, 8, BF16, 1.0),
                                                (1500, 4096, 4096, BF16, 0.7), (1, 17, 24, F32, 2.0)])
def test_shapes(R, V, stride, dtype, T):
    gu.log(f"[case] sample shapes R={R} V={V} stride={stride} dtype={dtype} T={T}")
    rng = np.random.default_rng(R + V)
    x = rng.normal(0, 2, (R, stride)).astype(np.float32)
    raw = synth.f32_to_bf16_bits(x) if dtype == BF16 else x
    _check_draws(raw, T, seed=R * 7 + 1, offset=V, vocab=V, what=f"shape {R}x{V}")


def test_special_values():
    """-inf logits never win while a finite one exists; a NaN logit wins its row (first NaN)."""
    gu.log("[case] sample special values")
    x = np.random.default_rng(3).normal(0, 1, (4, 64)).astype(np.float32)
    x[0, :] = -np.inf
    x[0, 40] = -5.0
    x[1, 10] = np.nan
    x[1, 50] = np.nan
    x[2, :] = -np.inf
    got = _check_draws(x, 1.0, seed=5, offset=5, what="special")
    assert got[0] == 40 and got[1] == 10 and got[2] == 0


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_special_values_across_loads(dtype):
    """Special logits in rows of several 16-byte loads per thread: the first NaN wins wherever it
    sits; +inf logits win (the first of them); +inf and -inf in one load of eight; a row of -inf
    with one finite logit; the ragged end of a row that is not a multiple of eight."""
    gu.log(f"[case] sample special values across loads dtype={dtype}")
    V = 4099  # (rows padded to 4104: a row's bytes must be a multiple of 16)
    x = np.random.default_rng(8).normal(0, 1, (6, 4104)).astype(np.float32)
    x[:, V:] = np.nan  # past the vocabulary: never read
    x[0, 3000] = np.nan
    x[0, 1000] = np.nan
    x[1, 2000] = np.inf
    x[1, 17] = np.inf
    x[2, 9] = np.inf
    x[2, 10] = -np.inf
    x[3, :V] = -np.inf
    x[3, 4097] = 0.0
    x[4, 4098] = np.nan
    x[5, 8:16] = np.array([np.inf, -np.inf, 0, 0, 0, 0, 0, 0], np.float32)
    x[5, 2] = np.nan
    raw = synth.f32_to_bf16_bits(x) if dtype == BF16 else x
    got = _check_draws(raw, 1.0, seed=21, offset=4, vocab=V, what="special across loads")
    assert got.tolist() == [1000, 17, 9, 4097, 4098, 2]


def test_law_and_noise():
    """The GPU draws follow softmax(z/T) (chi-square), repeat for the same (seed, offset) and
    change with the offset."""
    gu.log("[case] sample law")
    z = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 0.9, -2.0], np.float32)
    R = 40000
    rows = np.tile(z, (R, 1))
    for T in (0.5, 1.5):
        a = _gpu_sample(rows, T, seed=11, offset=1)
        _chi2_ok(np.bincount(a, minlength=8), _softmax(z / T), f"gpu law T={T}")
    a = _gpu_sample(rows, 1.0, seed=11, offset=1)
    b = _gpu_sample(rows, 1.0, seed=11, offset=1)
    c = _gpu_sample(rows, 1.0, seed=11, offset=2)
    assert (a == b).all() and (a != c).mean() > 0.5


def test_sampled_step_matches_oracle():
    """Draws plus sampled acceptance on the 8-sequence workload: acceptance, path, bonus and tokens
    bit-exact against the oracle's sampled acceptance of the same draws."""
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] sampled step c8")
    w = gu.cached_config("c8")
    d = gu.dev_workload(w)
    for T, off in ((1.0, 11), (0.3, 12)):
        tgt, _ = ev.node_sample(d["logits"], temperature=T, seed=2024, offset=off)
        acc = ev.sampled_accept(d["node_start"], d["parent"], d["draft"], tgt, max_nodes=w.max_nodes, vocab=w.vocab)
        torch.cuda.synchronize()
        draws = tgt.cpu().numpy()
        # the draws against the oracle's (near ties aside), then acceptance on those same draws
        assert np.array_equal(draws, _check_draws(w.logits, T, 2024, off, what=f"step T={T}"))
        ref = oracle.sampled_accept(w.node_start, w.parent, w.draft, draws, w.max_nodes, w.vocab)
        for k in ("accept_len", "accept_path", "bonus", "out_tokens"):
            assert np.array_equal(acc[k].cpu().numpy(), ref[k]), k


def test_argument_errors():
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] sample argument errors")
    x = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    for T in (0.0, -1.0, float("inf"), float("nan"), 1e-45):
        with pytest.raises(ev.EvError) as e:
            ev.node_sample(x, temperature=T, seed=1, offset=1)
        assert e.value.status == 2, T
