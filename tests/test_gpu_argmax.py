"""The decoder step's greedy argmax with planted exact ties.

The vocabulary projection is tied to the token embedding, so equal embedding
rows give bit-equal logits (every column goes through the same arithmetic).
Rows {3, 21, 40000} are set to c v and rows {4, 22, 40001} to -c v for a
large c, so on almost every batch row the maximum is one of these sets, tied
three ways: between blocks of one workgroup (21) and between workgroups
(40000); 3 and 4 share a 16-column block. (The two sets' logits are close to,
but not bitwise, negatives of each other: the MFMA's accumulation is not
sign-symmetric.) The argmax must be the lowest column of the winning set
(3 where its logit is at least that of 4, else 4) on every row where a planted
set holds the maximum, and on every row the first maximum of the logits the
step returned."""
import numpy as np
import pytest
import torch

from speech_recognition_amd.runtime import DecodeState, Whisper
from tests.gpu_util import need_gpu, say
from workload import CONFIGS, gen_normal, gen_prefill_lengths, gen_tokens, gen_weights

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("B", [64, 37])
def test_argmax_lowest_index_on_planted_ties(B):
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=1)
    W = gen_weights(DEV, dims)
    emb = W["decoder.token_embedding"]
    v = gen_normal(DEV, (dims.d_model,), dims.cfg_id, 9, 1)
    v = v / v.norm() * 400.0
    for r in (3, 21, 40000):
        emb[r] = v
    for r in (4, 22, 40001):
        emb[r] = -v
    m = Whisper(dims, list(W.values()))
    del W
    enc = gen_normal(DEV, (B, dims.n_audio_ctx, dims.d_model), dims.cfg_id, 5, 2, bf16=True).to(torch.bfloat16)
    cap = 64
    lengths0 = gen_prefill_lengths(DEV, dims.cfg_id, B, 32)
    st = DecodeState(dims, B, cap, None, torch.full((1, 2), 0.02), lengths0, enc=enc)
    toks = gen_tokens(DEV, dims.cfg_id, 2, B, dims.n_vocab)
    logits = torch.empty(B, dims.n_vocab, dtype=torch.float32, device=DEV)
    for t in range(2):
        m.decode_step(st, toks[t], logits)
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()
        am = st.argmax.cpu().numpy()
        assert np.isfinite(lg).all()
        for a, b in ((3, 21), (3, 40000), (4, 22), (4, 40001)):
            assert np.array_equal(lg[:, a], lg[:, b]), f"planted rows {a}, {b} differ"
        # rows whose planted logit is the maximum (all but those where v is
        # nearly orthogonal to the normalised activations)
        top = (np.maximum(lg[:, 3], lg[:, 4])[:, None] >= lg).all(axis=1)
        assert top.mean() >= 0.9, f"planted maximum on only {int(top.sum())} of {B} rows"
        want = np.where(lg[:, 3] >= lg[:, 4], 3, 4)
        bad = top & (am != want)
        assert not bad.any(), f"step {t}: argmax {am[bad][:4]} where {want[bad][:4]}"
        assert np.array_equal(am, np.argmax(lg, axis=1))
    assert np.array_equal(st.lengths.cpu().numpy(), lengths0.cpu().numpy() + 2)
    say(f"  B={B}: argmax is the lowest tied column on every row, 2 steps")
