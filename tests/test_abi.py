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
