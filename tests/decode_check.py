"""Comparators for the decoder-step parity tests.

The GPU and the oracle each keep their own fp8 KV cache; the oracle never
reads a value the GPU produced. The library's K/V debug hooks give the test
the fp32 values the GPU's codec was applied to (kv_pre), and let the test
hand the GPU the oracle's codes for the slots it appends (kv_force).

Two ways of running a case:
* forced (the parity gate): before each GPU step the oracle runs the same
  step on its own and its codes are forced into the GPU's appends, so at
  every layer both sides read the same cache. The fp8 cache turns a
  bf16-level difference in a quantised value into a whole e4m3 step when it
  sits near a rounding midpoint, and with few cached slots that step changes
  the attention output and every later layer; forcing keeps each layer's
  comparison to that layer's own arithmetic. Bars: logits and K/V within TOL,
  argmax equal unless tied, codes equal to the oracle's except at near-ties.
* independent: no forcing. The codec is exact on the GPU's own values, and
  the logits are within the oracle's own sensitivity: twice the distance
  between the oracle and the oracle run with its quantised K/V rounded to
  bf16 (never less than TOL).
"""
import numpy as np
import torch

from oracle import whisper_oracle as O
from speech_recognition_amd import _lib as L
from tests.gpu_util import TOL, rel_err

# Near-tie band of the code comparison, in units of the scaled value
# y = x / s: the kernel's code may differ from the oracle's only if it is the
# code of some value within delta of the oracle's y, where
#   delta = DELTA_REL * sqrt(3 l + 1) * rms(y over the row's H*64 values)
# at decoder layer l. The kernel's K / V carry an absolute error per row: the
# bf16 rounding (unit roundoff 2^-9) of the activations that feed them. At
# layer 0 that is the one rounding of the projection's own operands; by layer
# l the residual stream has also taken 3 l bf16-rounded sublayer outputs
# (self-attention, cross-attention, MLP per layer), whose independent errors
# add like a random walk. DELTA_REL = 8 * 2^-9 puts the band at eight times
# the unit roundoff per rounding. It is relative to the row's RMS, not to each
# element, because a per-element relative band is empty near zero.
DELTA_REL = 2.0 ** -6


class KvTrace:
    """Arms the K/V debug hooks on device buffers of n_layers x 2 x rows x d
    elements for the duration of a with-block: kv_pre always, kv_force when
    force=True (all entries -1, i.e. keep the kernel's code, until set)."""

    def __init__(self, n_layers, rows, d, force=False, device="cuda"):
        self.shape = (n_layers, 2, rows, d)
        self.buf = torch.full(self.shape, float("nan"), dtype=torch.float32, device=device)
        self.force = torch.full(self.shape, -1, dtype=torch.int16, device=device) if force else None

    def __enter__(self):
        L.whisper_debug_kv_arm(self.buf, self.force, self.buf.numel())
        return self

    def __exit__(self, *exc):
        L.whisper_debug_kv_disarm()
        return False

    def set_force(self, codes_by_row, rows_total):
        """codes_by_row: {activation row: [n_layers, 2, d] codes}; every other
        row keeps the kernel's own codes. rows_total: the call's activation
        rows (the buffer is indexed [n_layers][2][rows_total][d])."""
        n_layers, _, r_max, d = self.shape
        f = np.full((n_layers, 2, rows_total, d), -1, np.int16)
        for r, c in codes_by_row.items():
            f[:, :, r, :] = np.asarray(c, np.int16).reshape(n_layers, 2, d)
        self.force.view(-1)[:f.size].copy_(torch.from_numpy(f.reshape(-1)))

    def take(self, rows=None):
        """The last call's values as float64 [n_layers, 2, rows, d] (rows: that
        call's activation rows, default the buffer's); the buffer is refilled
        with NaN so a value a later call fails to write shows."""
        torch.cuda.synchronize()
        n_layers, _, r_max, d = self.shape
        rows = r_max if rows is None else rows
        assert rows <= r_max
        out = self.buf.view(-1)[:n_layers * 2 * rows * d].view(n_layers, 2, rows, d).cpu().numpy()
        self.buf.fill_(float("nan"))
        return out.astype(np.float64)


def check_codec_exact(kv_gpu, codes_gpu, scale, where):
    """The codes the GPU wrote are the codec applied to the GPU's own fp32
    values, bit for bit, without exception."""
    kv_gpu = np.asarray(kv_gpu, np.float64).reshape(-1)
    cg = np.asarray(codes_gpu, np.uint8).reshape(-1)
    assert np.isfinite(kv_gpu).all(), f"{where}: K/V debug values not written"
    bad = np.flatnonzero(O.e4m3_quantize(kv_gpu, scale) != cg)
    assert bad.size == 0, f"{where}: {bad.size} codes are not the codec of the kernel's values (first {bad[:4]})"


def check_kv_against_oracle(kv_gpu, kv_ref, codes_ref, scale, where, layer=0, kv_moved=None):
    """The GPU's fp32 K / V of one appended row (decoder layer `layer`) against
    the oracle's: within TOL, and the kernel's codes for them equal to the
    oracle's except at near-ties (the band above). kv_moved: the same K / V
    from an oracle run with a perturbation the kernels also carry (the fp8
    MLP sites' inputs rounded to bf16); the bar is then max(TOL, twice the
    distance it moved them) and the band also covers twice the largest
    distance it moved one value. Returns (differing codes, rel. error)."""
    kv_gpu = np.asarray(kv_gpu, np.float64).reshape(-1)
    kv_ref = np.asarray(kv_ref, np.float64).reshape(-1)
    co = np.asarray(codes_ref, np.uint8).reshape(-1)
    assert np.isfinite(kv_gpu).all(), f"{where}: K/V debug values not written"
    e = rel_err(kv_gpu, kv_ref)
    bar = TOL if kv_moved is None else max(TOL, 2.0 * rel_err(np.asarray(kv_moved).reshape(-1), kv_ref))
    assert e < bar, f"{where}: K/V before quantisation rel err {e:.3e} (bar {bar:.3e})"
    cg = O.e4m3_quantize(kv_gpu, scale)
    y = O.e4m3_pre_quant(kv_ref, scale).astype(np.float64)
    delta = DELTA_REL * np.sqrt(3 * layer + 1) * np.sqrt(np.mean(y * y))
    if kv_moved is not None:
        y_m = O.e4m3_pre_quant(np.asarray(kv_moved, np.float64).reshape(-1), scale).astype(np.float64)
        delta = max(delta, 2.0 * float(np.abs(y_m - y).max()))
    vlo = O.e4m3_value(O.e4m3_encode((y - delta).astype(np.float32)))
    vhi = O.e4m3_value(O.e4m3_encode((y + delta).astype(np.float32)))
    vg = O.e4m3_value(cg)
    diff = cg != co
    ok = ~diff | ((vg >= vlo) & (vg <= vhi))
    assert ok.all(), f"{where}: {int((~ok).sum())} codes differ from the oracle's outside the near-tie band"
    return int(diff.sum()), e


def gpu_codec_on_oracle_values(kv_ref_list, scale_list, codes_ref_list, device="cuda"):
    """The GPU codec (whisper_fp8_quantize) fed the oracle's own scaled fp32
    values y = fl32(x) * fl32(1 / s) at scale 1 must emit exactly the oracle's
    codes. One launch for a list of rows."""
    ys = [O.e4m3_pre_quant(k, s).reshape(-1) for k, s in zip(kv_ref_list, scale_list)]
    want = np.concatenate([np.asarray(c, np.uint8).reshape(-1) for c in codes_ref_list])
    y = torch.from_numpy(np.ascontiguousarray(np.concatenate(ys), dtype=np.float32)).to(device)
    one = torch.ones(4, dtype=torch.float32, device=device)
    c = torch.empty(y.numel(), dtype=torch.uint8, device=device)
    L.whisper_fp8_quantize(y, L.WHISPER_F32, y.numel(), one, c, None)
    torch.cuda.synchronize()
    return np.array_equal(c.cpu().numpy(), want)


def check_logits_argmax(lg_gpu, am_gpu, lg_ref, rows, tag, tol=TOL):
    """Per row: logits within tol (max-normalised); argmax equal to the
    oracle's unless the row is tied (oracle top-1 - top-2 gap at most twice
    the row's largest logit difference). The argmax is also checked exactly
    against the GPU's own logits: the first largest value of the row.
    Returns the number of tied rows."""
    n_tied = 0
    for b in rows:
        assert am_gpu[b] == int(np.argmax(lg_gpu[b])), f"{tag} row {b}: argmax is not the first max of its logits"
        e = rel_err(lg_gpu[b], lg_ref[b])
        assert e < tol, f"{tag} row {b}: logits rel err {e:.3e} (bar {tol:.3e})"
        if O.top2_gap(lg_ref[b]) <= 2 * np.abs(lg_gpu[b] - lg_ref[b]).max():
            n_tied += 1
            continue
        assert am_gpu[b] == int(O.greedy_token(lg_ref[b])), f"{tag} row {b}: argmax differs"
    return n_tied
