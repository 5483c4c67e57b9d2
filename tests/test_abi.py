"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes come out as documented, and bad arguments are
rejected before any launch (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from speech_recognition_amd import _lib as L
from workload import CONFIGS, weight_specs

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "whisper_mi355x.h")


def header_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(whisper_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_header_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    syms = header_symbols()
    assert len(syms) >= 18
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(L.EXPORTS) == syms


def test_weight_count_matches_canonical_order():
    for name, d in CONFIGS.items():
        assert L.whisper_weight_count(d) == len(weight_specs(d)), name


def test_sizes():
    d = CONFIGS["v3_decode"]
    assert L.whisper_packed_weights_size(d) > 2 * (51866 * 1280 + 32 * 26_000_000) * 0.9
    ws = L.whisper_workspace_size(d, 64, L.WS_DECODE)
    assert ws >= 64 * 51866 * 4
    enc = CONFIGS["v3_encoder"]
    assert L.whisper_workspace_size(enc, 8, L.WS_ENCODE) >= 8 * 1500 * 5120 * 2
    assert L.whisper_workspace_size(enc, 0, L.WS_ENCODE) == 0
    assert L.whisper_fp8_workspace_size() == 4096
    assert L.whisper_attention_decode_cross_workspace_size(64, 20, 1500) == 0  # single pass, no partials


def test_bad_dims_rejected():
    bad = CONFIGS["v3_layer"].with_(n_heads=19)
    assert L.whisper_packed_weights_size(bad) == 0
    with pytest.raises(L.WhisperError) as e:
        L.whisper_encode(bad, 16, 16, 1, 16, 16, 1 << 20, stream=0)
    assert e.value.status == 2 and "n_heads" in str(e.value)


def test_null_and_alignment_rejected():
    d = CONFIGS["v3_layer"]
    with pytest.raises(L.WhisperError) as e:
        L.whisper_encode(d, None, 16, 1, 16, 16, 1 << 40, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.WhisperError) as e:
        L.whisper_encode(d, 16, 17, 1, 16, 16, 1 << 40, stream=0)
    assert e.value.status == 4


def test_workspace_too_small_rejected():
    d = CONFIGS["v3_encoder"]
    with pytest.raises(L.WhisperError) as e:
        L.whisper_encode(d, 16, 16, 8, 16, 16, 1024, stream=0)
    assert e.value.status == 5 and "need" in str(e.value)


def test_decode_step_validation():
    d = CONFIGS["v3_decode"]
    with pytest.raises(L.WhisperError) as e:
        L.whisper_decode_step(d, 16, 64, 5000, 16, 16, 16, 16, 16, None, 16, None, 16, 1 << 40, stream=0)
    assert e.value.status == 2
    enc_only = CONFIGS["v3_layer"]
    with pytest.raises(L.WhisperError) as e:
        L.whisper_decode_step(enc_only, 16, 64, 672, 16, 16, 16, 16, 16, None, 16, None, 16, 1 << 40, stream=0)
    assert e.value.status == 2


def test_kernel_call_validation():
    with pytest.raises(L.WhisperError) as e:
        L.whisper_linear(L.WHISPER_BF16, 16, 8, 16, None, 10, 10, 100, 0, 16, stream=0)
    assert e.value.status == 2  # K % 64
    with pytest.raises(L.WhisperError) as e:
        L.whisper_linear(L.WHISPER_BF16, 16, 256, 16, None, 200, 10, 256, 0, 16, path=2, stream=0)
    assert e.value.status == 2  # skinny needs M <= 128
    with pytest.raises(L.WhisperError) as e:
        L.whisper_fp8_quantize(16, L.WHISPER_BF16, 10, None, 16, None, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.WhisperError) as e:
        L.whisper_fp8_quantize(16, L.WHISPER_BF16, 10, None, 16, 16, 16, 100, stream=0)
    assert e.value.status == 5
    with pytest.raises(L.WhisperError) as e:  # unknown fp8 format
        L.whisper_fp8_quantize(16, L.WHISPER_BF16, 10, 16, 16, None, stream=0, fmt=2)
    assert e.value.status == 1
    with pytest.raises(L.WhisperError) as e:
        L.whisper_fp8_dequantize(16, 10, 16, 16, L.WHISPER_F32, stream=0, fmt=-1)
    assert e.value.status == 1
    d = CONFIGS["v3_decode"]
    with pytest.raises(L.WhisperError) as e:
        L.whisper_decode_step_xq(d, 16, 64, 672, 16, 16, 16, 16, 16, 16, None, 16, None, 16, 1 << 40, stream=0,
                                 cross_format=7)
    assert e.value.status == 1
    with pytest.raises(L.WhisperError) as e:
        L.whisper_attention_decode_self(L.WHISPER_BF16, 16, 4, 20, 5000, 16, 16, 16, 16, 16, stream=0)
    assert e.value.status == 2
    assert L.whisper_status_string(6) == "KV cache capacity exceeded"


def test_chunk_plan_host_logic_matches_oracle():
    """whisper_chunk_plan is host arithmetic: its plan equals the oracle's for
    strides with and without overlap; invalid strides are rejected."""
    from oracle import whisper_oracle as O
    for n in (1, 479999, 480000, 480001, 1_200_000, 43_200_000):
        for stride in (480000, 400000, 320000, 160160):
            count, plan = L.whisper_chunk_plan(n, stride)
            assert count == len(plan) and plan == O.chunk_plan(n, stride), (n, stride)
    for bad in ((0, 400000), (1000, 0), (1000, 480160), (1000, 1000)):
        with pytest.raises(L.WhisperError):
            L.whisper_chunk_plan(*bad)
    # plan entries are int32: the longest recording whose chunk starts fit is
    # accepted, one sample more is rejected (about 37 h at 16 kHz)
    lib = L.lib()
    assert lib.whisper_chunk_plan(2**31 - 1, 480000, None, 0) == 1 + -(-(2**31 - 1 - 480000) // 480000)
    assert lib.whisper_chunk_plan(2**31, 480000, None, 0) == 0
    assert lib.whisper_chunk_plan(2**40, 160, None, 0) == 0


def _al(n):
    return (n + 255) // 256 * 256


def test_plan_batch_host_logic():
    """whisper_plan_batch is host arithmetic over the size queries: the plan
    fits the budget, one more chunk does not, the stage sums follow the
    documented schedule, and the footprint grows with the batch."""
    G = 1 << 30
    full = CONFIGS["v3_decode"].with_(n_enc_layers=32)
    # the showcase page's example cap: 24 GB on a shared card; this footprint
    # admits exactly the 64-chunk batch of the large-v3 decode workload
    assert L.whisper_plan_batch(full, 24 * G, 672, 4, False, True)["batch"] == 64
    prev = 0
    for budget in (6 * G, 24 * G, 80 * G, 288 * G):
        for fp8 in (False, True):
            for P, logits in ((0, False), (4, True)):
                p = L.whisper_plan_batch(full, budget, 672, P, fp8, logits)
                B = p["batch"]
                assert 1 <= B and p["total"] <= budget
                nxt = L.whisper_plan_batch(full, 1 << 62, 672, P, fp8, logits, max_batch=B + 1)
                assert nxt["batch"] == B + 1 and nxt["total"] > budget
                Lh, H, T, D, e = 32, 20, 1500, 1280, 2
                assert p["weights"] == _al(L.whisper_packed_weights_size(full))
                ws = max(L.whisper_workspace_size(full, B, k) for k in (L.WS_LOGMEL, L.WS_ENCODE, L.WS_DECODE))
                ws = max(ws, L.whisper_workspace_size(full, B * max(P, 1), L.WS_DECODE))
                if fp8:
                    ws = max(ws, _al(L.whisper_fp8_workspace_size()))
                assert p["workspace"] == ws
                assert p["audio"] == _al(B * 480000 * 4) and p["mel"] == _al(B * 128 * 3000 * 4)
                assert p["encoder_out"] == _al(B * T * D * e)
                assert p["cross_kv"] == _al(Lh * 2 * B * H * T * 64 * e)
                assert p["cross_codes"] == (_al(Lh * 2 * B * H * T * 64) + _al(Lh * 2 * 4) if fp8 else 0)
                assert p["kv_cache"] == _al(Lh * 2 * B * H * 672 * 64)
                assert p["logits"] == (_al(B * 51866 * 4) if logits else 0)
                st = p["stage"]
                assert st["logmel"] == p["audio"] + p["mel"]
                assert st["encode"] == p["mel"] + p["encoder_out"]
                assert st["cross_kv"] == p["encoder_out"] + p["cross_kv"]
                assert st["quantise"] == (p["cross_kv"] + p["cross_codes"] if fp8 else 0)
                assert st["decode"] == ((p["cross_codes"] if fp8 else p["cross_kv"]) + p["kv_cache"]
                                        + p["decode_state"] + p["logits"])
                assert p["total"] == p["weights"] + p["workspace"] + max(st.values())
                assert st[p["peak_stage"]] == max(st.values())
        b24 = L.whisper_plan_batch(full, budget, 672)["batch"]
        assert b24 > prev
        prev = b24
    # the prefill bound B * P <= 4096 and max_batch cap
    assert L.whisper_plan_batch(full, 1 << 62, 672, 64)["batch"] == 64
    assert L.whisper_plan_batch(full, 1 << 62, 672, 0, max_batch=7)["batch"] == 7
    with pytest.raises(L.WhisperError) as e:
        L.whisper_plan_batch(full, 3 * G, 672)
    assert e.value.status == 6
    with pytest.raises(L.WhisperError) as e:
        L.whisper_plan_batch(CONFIGS["v3_decode"], 24 * G, 672)
    assert e.value.status == 2
    with pytest.raises(L.WhisperError) as e:
        L.whisper_plan_batch(full, 24 * G, 5000)
    assert e.value.status == 2


def test_fp8_encoder_entry_validation():
    """Host checks of the mixed_fp8 entry points (no launch happens)."""
    v3 = CONFIGS["v3_decode"].with_(n_enc_layers=32)
    tiny = CONFIGS["tiny_f32"]
    # packed size: per encoder layer 3 d^2 + 2 d f bytes of codes (256-aligned),
    # then 8 scales per encoder layer; per decoder layer the MLP's two weights
    # as codes and its first bias as fp32, then 2 scales per decoder layer
    d, f = 1280, 5120
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    enc = 32 * (al(3 * d * d) + al(f * d) + al(d * f)) + al(32 * 8 * 4)
    dec = 32 * (al(f * d) + al(d * f) + al(f * 4)) + al(32 * 2 * 4)
    assert L.whisper_packed_weights_fp8_size(v3) == enc + dec
    # no encoder layers: the scale block keeps one layer's slot
    assert L.whisper_packed_weights_fp8_size(CONFIGS["v3_decode"]) == al(8 * 4) + dec
    ws = L.whisper_workspace_size(v3, 2, L.WS_ENCODE_FP8)
    assert ws > L.whisper_workspace_size(v3, 2, L.WS_ENCODE)
    with pytest.raises(L.WhisperError) as e:  # fp32 model
        L.whisper_encode_fp8(tiny, 16, 16, 16, 1, 16, 16, 1 << 40, stream=0)
    assert e.value.status == 3
    with pytest.raises(L.WhisperError) as e:  # workspace too small
        L.whisper_encode_fp8(v3, 16, 16, 16, 2, 16, 16, ws - 1, stream=0)
    assert e.value.status == 5
    with pytest.raises(L.WhisperError) as e:  # layer range
        L.whisper_encode_layers_fp8(v3, 16, 16, 16, 1, 3, 40, False, 16, 16, 1 << 40, stream=0)
    assert e.value.status == 2
    with pytest.raises(L.WhisperError) as e:  # pack workspace below whisper_fp8_workspace_size()
        L.whisper_pack_weights_fp8(v3, [16] * L.whisper_weight_count(v3), 16, 16, 8, stream=0)
    assert e.value.status == 5
    # whisper_gemm_fp8 shape rules: K % 256, K >= 512, N % 256, ldc, rows_per_scale
    ok = dict(M=100, K=512, rps=256, N=256, ldc=256)
    for bad in (dict(K=384), dict(K=256), dict(N=200), dict(ldc=200), dict(ldc=260), dict(rps=100)):
        a = {**ok, **bad}
        with pytest.raises(L.WhisperError) as e:
            L.whisper_gemm_fp8(16, a["M"], a["K"], 16, a["rps"], 16, a["N"], 16, None, False, 16, a["ldc"], stream=0)
        assert e.value.status == 2, bad
    with pytest.raises(L.WhisperError) as e:
        L.whisper_gemm_fp8(16, 0, 512, 16, 256, 16, 256, 16, None, False, 16, 256, stream=0)
    assert e.value.status == 1


def test_decode_mlp_fp8_validation():
    """Host checks of whisper_decode_mlp_fp8 (no launch happens)."""
    ws = L.whisper_decode_mlp_fp8_workspace_size(64, 1280, 5120)
    # at least both weights' codes, x tiles, quantised rows and hidden rows
    assert ws >= 2 * 1280 * 5120 + 64 * 1280 * 4 + 64 * 1280 * 2 + 64 * 5120 * 2
    for bad in ((0, 1280, 5120), (4097, 1280, 5120), (64, 1000, 5120), (64, 2080, 5120), (64, 1280, 5000),
                (64, 1280, 4080)):
        assert L.whisper_decode_mlp_fp8_workspace_size(*bad) == 0, bad
        with pytest.raises(L.WhisperError) as e:
            L.whisper_decode_mlp_fp8(*bad, 16, 16, 16, 16, 16, 16, 16, ws=16, ws_bytes=1 << 40, stream=0)
        assert e.value.status == 2, bad
    with pytest.raises(L.WhisperError) as e:  # workspace too small
        L.whisper_decode_mlp_fp8(64, 1280, 5120, 16, 16, 16, 16, 16, 16, 16, ws=16, ws_bytes=ws - 1, stream=0)
    assert e.value.status == 5
    with pytest.raises(L.WhisperError) as e:  # NULL weight
        L.whisper_decode_mlp_fp8(64, 1280, 5120, 16, 16, 16, None, 16, 16, 16, ws=16, ws_bytes=ws, stream=0)
    assert e.value.status == 1


def test_decode_linear_validation():
    """Host checks of whisper_decode_linear (no launch happens): modes, shape
    rules of the split-K and QKV forms, workspace size."""
    M, N, K = 64, 1280, 1280
    ws = L.whisper_decode_linear_workspace_size(L.DEC_LN_STORE, M, N, K)
    # packed weight (rows padded to 16), c1, b2 and the 16-row x tiles
    assert ws >= N * K * 2 + 2 * N * 4 + M * K * 4
    assert L.whisper_decode_linear_workspace_size(L.DEC_RESID_SPLITK, M, 1280, 5120) > \
        L.whisper_decode_linear_workspace_size(L.DEC_RESID, M, 1280, 5120)  # + partials and counters
    assert L.whisper_decode_linear_workspace_size(7, M, N, K) == 0
    assert L.whisper_decode_linear_workspace_size(L.DEC_LN_STORE, 5000, N, K) == 0
    assert L.whisper_decode_linear_workspace_size(L.DEC_LN_STORE, M, N, 100) == 0

    def call(mode, M=64, N=1280, K=1280, ws_bytes=1 << 40, **kw):
        args = dict(x=16, a=16, w=16, bias=None, gamma=16, beta=16, y=16, kv_cache=16, kv_scales=16, lengths=16,
                    kv_cap=672, dev_error=None, ws=16)
        args.update(kw)
        L.whisper_decode_linear(mode, M, N, K, args["x"], args["a"], args["w"], args["bias"], args["gamma"],
                                args["beta"], args["y"], args["kv_cache"], args["kv_scales"], args["lengths"],
                                args["kv_cap"], args["dev_error"], args["ws"], ws_bytes, stream=0)

    for kw, status in ((dict(mode=9), 1), (dict(mode=0, M=0), 1), (dict(mode=0, M=4097), 1),
                       (dict(mode=0, K=100), 2), (dict(mode=4, N=1000), 2),
                       (dict(mode=5, N=1280, K=1280), 2), (dict(mode=5, N=1200, K=5120), 2),
                       (dict(mode=3, N=3000), 2), (dict(mode=3, N=3840, kv_cap=0), 2),
                       (dict(mode=0, gamma=None), 1), (dict(mode=4, a=None), 1), (dict(mode=0, x=24), 4),
                       (dict(mode=3, N=3840, lengths=None), 1), (dict(mode=0, ws_bytes=1024), 5)):
        with pytest.raises(L.WhisperError) as e:
            call(**kw)
        assert e.value.status == status, kw


def test_debug_kv_hook_checked_before_launch():
    """The K/V debug hook: NULL or misaligned buffers are rejected, and a call
    whose trace would overflow the armed buffer fails with WORKSPACE before
    launching anything; disarming restores normal validation."""
    with pytest.raises(L.WhisperError) as e:
        L.whisper_debug_kv_arm(None, None, 10)
    assert e.value.status == 1
    with pytest.raises(L.WhisperError) as e:
        L.whisper_debug_kv_arm(18, None, 10)
    assert e.value.status == 4
    with pytest.raises(L.WhisperError) as e:
        L.whisper_debug_kv_arm(None, 17, 10)
    assert e.value.status == 4
    d = CONFIGS["v3_decode"]
    ws = L.whisper_workspace_size(d, 4, L.WS_DECODE)
    L.whisper_debug_kv_arm(16, 32, 32 * 2 * 4 * 1280 - 1)  # one element short of 32 layers x K, V x 4 rows
    try:
        with pytest.raises(L.WhisperError) as e:
            L.whisper_decode_step(d, 16, 4, 672, 16, 16, 16, 16, 16, None, 16, None, 16, ws, stream=0)
        assert e.value.status == 5 and "debug" in str(e.value)
        with pytest.raises(L.WhisperError) as e:
            L.whisper_decode_linear(L.DEC_LN_QKV, 4096, 3840, 1280, 16, 16, 16, None, 16, 16, 16, 16, 16, 16, 672,
                                    None, 16, 1 << 40, stream=0)
        assert e.value.status == 5
    finally:
        L.whisper_debug_kv_disarm()


def test_decode_step_noalloc_host_checks():
    """The allocation-free step needs logits and a batch whose workspace fits
    the library's scratch; both are checked before any launch."""
    d = CONFIGS["v3_decode"]
    with pytest.raises(L.WhisperError) as e:  # logits NULL
        L.whisper_decode_step_noalloc(d, 16, 64, 672, 16, 16, 16, 16, 16, None, 16, None, stream=0)
    assert e.value.status == 1
    with pytest.raises(L.WhisperError) as e:  # 160 rows need more than the 8 MiB scratch
        L.whisper_decode_step_noalloc(d, 16, 160, 672, 16, 16, 16, 16, 16, 16, 16, None, stream=0)
    assert e.value.status == 5 and "scratch" in str(e.value)
