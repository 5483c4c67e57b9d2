"""GPU parity of the decoder-step projections (whisper_decode_linear: the
LayerNorm-folded GEMMs with their store / GELU / fp32 / QKV + fp8-append
epilogues and the residual GEMMs, plain and split-K) against the oracle's
LayerNorm + linear, at the batch-64 large-v3 shapes and a ragged row count.
Every output buffer is surrounded by canary bytes that must survive."""
import numpy as np
import pytest
import torch

from oracle import whisper_oracle as O
from speech_recognition_amd import _lib as L
from tests.decode_check import KvTrace, check_codec_exact, check_kv_against_oracle
from tests.gpu_util import TOL, host, need_gpu, rel_err, say
from workload import gen_normal

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 1024  # canary elements on each side of an output


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def guarded(n, dtype, fill):
    """A device buffer of n elements inside canaries; returns (whole, view)."""
    whole = torch.full((n + 2 * PAD,), fill, dtype=dtype, device=DEV)
    return whole, whole[PAD:PAD + n]


def canaries_intact(whole, fill):
    return bool(torch.all(whole[:PAD] == fill)) and bool(torch.all(whole[-PAD:] == fill))


def inputs(M, N, K, seed, mean_rows=()):
    """Residual rows x [M, K] (rows in mean_rows shifted by 50 standard
    deviations: the folded form's hard case), bf16 weights [N, K], bias,
    LayerNorm affine."""
    x = gen_normal(DEV, (M, K), 11, 6, seed)
    for r in mean_rows:
        x[r] = 50.0 + x[r]
    w = gen_normal(DEV, (N, K), 11, 0, seed, std=0.02, bf16=True)
    bias = gen_normal(DEV, (N,), 11, 0, seed + 1, std=0.02)
    gamma = 1.0 + gen_normal(DEV, (K,), 11, 0, seed + 2, std=0.1)
    beta = gen_normal(DEV, (K,), 11, 0, seed + 3, std=0.1)
    return x, w, bias, gamma, beta


def ws_for(mode, M, N, K):
    n = L.whisper_decode_linear_workspace_size(mode, M, N, K)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV), n


@pytest.mark.parametrize("mode,M,N,K", [
    (L.DEC_LN_STORE, 64, 1280, 1280),    # cross-attention query
    (L.DEC_LN_STORE, 37, 1280, 1280),    # ragged rows
    (L.DEC_LN_GELU, 64, 5120, 1280),     # MLP up-projection + GELU
    (L.DEC_LN_F32, 64, 51866, 1280),     # vocabulary projection, fp32 logits
    (L.DEC_LN_F32, 5, 51866, 1280),
])
def test_decode_linear_layernorm_folded(mode, M, N, K):
    say(f"decode_linear mode {mode} M={M} N={N} K={K}")
    mean_rows = (0, M - 1)
    x, w, bias, gamma, beta = inputs(M, N, K, 100 + mode, mean_rows)
    f32 = mode == L.DEC_LN_F32
    whole, y = guarded(M * N, torch.float32 if f32 else torch.bfloat16, -3.0)
    ws, nws = ws_for(mode, M, N, K)
    L.whisper_decode_linear(mode, M, N, K, x, None, w, bias, gamma, beta, y, ws=ws, ws_bytes=nws)
    torch.cuda.synchronize()
    assert canaries_intact(whole, -3.0), "write outside y"
    got = host(y).reshape(M, N)
    ref = O.linear(O.layer_norm(host(x), host(gamma), host(beta)), host(w), host(bias))
    if mode == L.DEC_LN_GELU:
        ref = O.gelu(ref)
    errs = [rel_err(got[r], ref[r]) for r in range(M)]
    say(f"  max row rel err {max(errs):.2e} (rows with mean 50 sd: {[f'{errs[r]:.1e}' for r in mean_rows]})")
    assert max(errs) < TOL
    if f32:  # the same argmax where not tied
        for r in range(M):
            if O.top2_gap(ref[r]) > 2 * np.abs(got[r] - ref[r]).max():
                assert int(np.argmax(got[r])) == int(O.greedy_token(ref[r])), r


def test_decode_linear_qkv_append():
    """The self-attention projection: the query in bf16, the key and value
    appended as e4m3 codes at slot lengths[m]. Codes are the codec of the
    kernel's own fp32 values (debug hook), those values match the oracle's,
    every other cache byte keeps its canary value, and a row whose slot is
    past the capacity sets the error word and writes nothing."""
    M, K, cap = 64, 1280, 672
    N, H = 3 * K, K // 64
    say(f"decode_linear QKV + fp8 append M={M} K={K} cap={cap}")
    x, w, bias, gamma, beta = inputs(M, N, K, 200, (3,))
    lengths = torch.randint(0, cap, (M,), generator=torch.Generator().manual_seed(4), dtype=torch.int32)
    lengths[5] = cap          # past the capacity: no write, error word set
    lengths[6] = cap - 1      # the last slot
    lengths[7] = 0
    scales = torch.tensor([0.004, 0.006], dtype=torch.float32, device=DEV)
    cache = torch.full((2, M, H, cap, 64), 0x5A, dtype=torch.uint8, device=DEV)
    qw, q = guarded(M * K, torch.bfloat16, -3.0)
    err = torch.zeros(4, dtype=torch.int32, device=DEV)
    ws, nws = ws_for(L.DEC_LN_QKV, M, N, K)
    with KvTrace(1, M, K) as tr:
        L.whisper_decode_linear(L.DEC_LN_QKV, M, N, K, x, None, w, bias, gamma, beta, q, cache, scales,
                                lengths.to(DEV), cap, err, ws, nws)
        kv_g = tr.take()
    assert int(err[0].item()) == 6
    assert canaries_intact(qw, -3.0)
    ref = O.linear(O.layer_norm(host(x), host(gamma), host(beta)), host(w), host(bias))
    assert rel_err(host(q).reshape(M, K), ref[:, :K]) < TOL
    c = cache.cpu().numpy()
    ln = lengths.numpy()
    sc = scales.cpu().numpy()
    written = np.zeros(c.shape, bool)
    flips = 0
    for m in range(M):
        for kv in range(2):
            if ln[m] >= cap:
                continue
            written[kv, m, :, ln[m], :] = True
            x_ref = ref[m, K * (1 + kv):K * (2 + kv)].reshape(H, 64)
            check_codec_exact(kv_g[0, kv, m], c[kv, m, :, ln[m], :], sc[kv], f"row {m} kv {kv}")
            nd, _ = check_kv_against_oracle(kv_g[0, kv, m], x_ref, O.e4m3_quantize(x_ref, sc[kv]), sc[kv],
                                            f"row {m} kv {kv}")
            flips += nd
    assert np.all(c[~written] == 0x5A), "cache bytes outside the appended slots changed"
    say(f"  codes differing from the oracle's at near-ties: {flips} of {2 * (M - 1) * K}")


@pytest.mark.parametrize("mode,M,N,K", [
    (L.DEC_RESID, 64, 1280, 1280),         # self / cross out-projection
    (L.DEC_RESID, 21, 1280, 1280),
    (L.DEC_RESID_SPLITK, 64, 1280, 5120),  # MLP down-projection, split-K over 4 workgroups
    (L.DEC_RESID_SPLITK, 50, 1280, 5120),
])
def test_decode_linear_residual(mode, M, N, K):
    say(f"decode_linear residual mode {mode} M={M} N={N} K={K}")
    a = gen_normal(DEV, (M, K), 12, 6, mode, std=0.5, bf16=True).to(torch.bfloat16)
    w = gen_normal(DEV, (N, K), 12, 0, mode, std=0.02, bf16=True)
    bias = gen_normal(DEV, (N,), 12, 0, mode + 10, std=0.02)
    xw, x = guarded(M * N, torch.float32, -3.0)
    x.copy_(gen_normal(DEV, (M * N,), 12, 6, mode + 20))
    x0 = host(x).reshape(M, N)
    ws, nws = ws_for(mode, M, N, K)
    for rep in range(2):  # twice in a row: the split-K tile counters are left at zero
        x.copy_(torch.from_numpy(x0.reshape(-1).astype(np.float32)).to(DEV))
        L.whisper_decode_linear(mode, M, N, K, x, a, w, bias, None, None, None, ws=ws, ws_bytes=nws)
        torch.cuda.synchronize()
        assert canaries_intact(xw, -3.0)
        delta = host(x).reshape(M, N) - x0
        ref = O.linear(host(a), host(w), host(bias))
        e = max(rel_err(delta[r], ref[r]) for r in range(M))
        assert e < TOL, (rep, e)
    say(f"  max row rel err of the added block {e:.2e}")
