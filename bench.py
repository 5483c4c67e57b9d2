#!/usr/bin/env python3
"""Throughput of the Whisper large-v3 hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
64 chunks of 30 s of 16 kHz audio -> GPU log-mel -> 32-layer encoder ->
224 teacher-forced decoder steps at batch 64 over an fp8 e4m3 self-KV cache
prefilled to seeded lengths U{1..448} (capacity 672), the cross-attention of
each decoder layer computed from the encoder output in its absorbed form
(whisper_decode_step_enc: no cross K/V are formed). Random N(0, 0.02)
weights, synthetic tones + noise; every input is resident in HBM before the
timed region.

Prints one JSON line: value = RTFx (audio seconds per wall second) of the
whole step, plus decode tokens/s, per-stage times, the roofline of the
dominant kernel (decoder cross-attention over the encoder output,
HBM-bound) timed with HIP events on its own stream inside the timed region,
and the CPU oracle timed on a bounded sample on the host cores.
"""
import argparse
import json
import os
import sys
import time

AUDIO_S = 30.0
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--decode-steps", type=int, default=224)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-probes", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the MFMA and HBM ceilings")
    ap.add_argument("--no-long-form", action="store_true",
                    help="skip the 45-minute long-form leg (turbo shape, batch 90; reported apart from value)")
    ap.add_argument("--no-fp8-encoder", "--no-mixed-fp8", action="store_true", dest="no_fp8_encoder",
                    help="skip the extra step with the mixed_fp8 sites (encoder QKV and FFN, decoder FFN in E4M3)")
    ap.add_argument("--no-fp8-cross", action="store_true",
                    help="skip the extra steps through explicit cross-attention K/V (bf16, fp8 e4m3, fp8 e5m2; "
                         "reported apart from value)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE / WRITE_SIZE, copy-calibrated), or None when that
    summary is missing or the kernel's sources changed since it was taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{kernel.split('_kernel')[0]}_hbm_counters.md")
    try:
        text = open(path).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        h = hashlib.sha256()
        for f in rec["sources"]:
            with open(os.path.join(here, f), "rb") as fh:
                h.update(fh.read())
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if rec.get("kernel") != kernel or h.hexdigest() != rec.get("source_sha256"):
        return None
    return int(rec["traffic_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by independent 30 s chunks with no exchange step)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from speech_recognition_amd import _lib as L
    from speech_recognition_amd.runtime import DecodeState, Whisper
    from workload import CONFIGS, gen_audio_tones, gen_prefill_kv, gen_prefill_lengths, gen_tokens, gen_weights

    DEV = "cuda"
    B, TD = args.batch, args.decode_steps
    dims = CONFIGS["v3_decode"].with_(name="large_v3", n_enc_layers=32)
    H, d, T, Ldec = dims.n_heads, dims.d_model, dims.n_audio_ctx, dims.n_dec_layers
    cap, prefill_max = 672, 448

    t0 = time.time()
    W = gen_weights(DEV, dims)
    model = Whisper(dims, list(W.values()), mixed_fp8=not args.no_fp8_encoder)
    torch.cuda.synchronize()
    del W
    torch.cuda.empty_cache()
    log(f"weights packed ({L.whisper_packed_weights_size(dims) / 1e9:.2f} GB) in {time.time() - t0:.1f}s")

    audio = gen_audio_tones(DEV, dims.cfg_id, B)
    lengths0 = gen_prefill_lengths(DEV, dims.cfg_id, B, prefill_max)
    tokens = gen_tokens(DEV, dims.cfg_id, TD, B, dims.n_vocab)
    mel = torch.empty(B, dims.n_mels, 3000, dtype=torch.float32, device=DEV)
    enc = torch.empty(B, T, d, dtype=torch.bfloat16, device=DEV)
    logits = torch.empty(B, dims.n_vocab, dtype=torch.float32, device=DEV)
    state = DecodeState(dims, B, cap, None, torch.ones(Ldec, 2), lengths0, enc=enc)
    fp8_ws = torch.empty(L.whisper_fp8_workspace_size(), dtype=torch.uint8, device=DEV)
    for l in range(Ldec):
        for kv in range(2):
            x = gen_prefill_kv(DEV, dims.cfg_id, l, kv, B, H, prefill_max)
            codes = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
            # per-layer scale from the prefill maximum, computed on the device
            L.whisper_fp8_quantize(x, L.WHISPER_F32, x.numel(), None, codes,
                                   state.kv_scales[l, kv:kv + 1].data_ptr(), fp8_ws, fp8_ws.numel())
            state.kv_cache[l, kv, :, :, :prefill_max, :] = codes
            del x, codes
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s; encoder output {enc.numel() * 2 / 1e9:.2f} GB, "
        f"KV cache {state.kv_cache.numel() / 1e9:.2f} GB")

    def run_step(ev=None):
        if ev:
            ev[0].record()
        model.logmel(audio, out=mel)
        if ev:
            ev[1].record()
        model.encode(mel, out=enc)
        if ev:
            ev[2].record()
        state.lengths.copy_(lengths0)
        for t in range(TD):
            model.decode_step(state, tokens[t], logits)
        if ev:
            ev[3].record()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    assert int(state.dev_error[0].item()) == 0
    log(f"warmup done at {time.time() - t0:.1f}s")

    # dominant kernel: decoder cross-attention over the encoder output, events
    # on the launch stream inside the timed region
    n_ev = min(2048, Ldec * TD * args.steps)
    k_start = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    k_stop = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in k_start + k_stop:
        e.record()
    stage_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()

    L.whisper_profile_arm(L.PROF_DECODE_CROSS_ATTENTION, k_start, k_stop)
    torch.cuda.synchronize()
    t_begin = time.perf_counter()
    for s in range(args.steps):
        run_step(stage_ev[s])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    n_rec = L.whisper_profile_disarm()
    elapsed = t_end - t_begin
    ms_step = elapsed / args.steps * 1e3

    stage_names = ["logmel", "encode", "decode"]
    stage_ms = {n: float(np.mean([stage_ev[s][i].elapsed_time(stage_ev[s][i + 1]) for s in range(args.steps)]))
                for i, n in enumerate(stage_names)}
    cross_ms = float(np.mean([k_start[i].elapsed_time(k_stop[i]) for i in range(n_rec)]))
    # per batch row and layer: the encoder output (T x d bf16) read once, the
    # absorbed query q' (H x d bf16) in, the per-head weighted sum u (H x d bf16) out
    cross_bytes = B * (T * d * 2 + 2 * H * d * 2)
    cross_gbs = cross_bytes / (cross_ms * 1e-3) / 1e9
    enc_flop = B * (2 * 3000 * 3 * dims.n_mels * d + 2 * 1500 * 3 * d * d) + B * 32 * (
        2 * T * d * 3 * d + 2 * T * d * d + 2 * 2 * T * d * dims.d_ffn + 4 * T * T * d)
    rtfx = B * AUDIO_S / (elapsed / args.steps)
    decode_tok_s = B * TD / (stage_ms["decode"] * 1e-3)
    log(f"timed {args.steps} steps: {ms_step:.1f} ms/step, RTFx {rtfx:.0f}, stages {stage_ms}")
    log(f"cross-attention: {n_rec} launches timed, {cross_ms * 1e3:.1f} us avg, {cross_gbs:.0f} GB/s")

    peaks = None if args.no_peaks else measured_peaks(L, torch)
    lf = None if args.no_long_form else long_form(L, torch, Whisper, DecodeState)

    fp8e = None
    if not args.no_fp8_encoder:
        fp8e = fp8_encoder_step(model, audio, mel, enc, state, tokens, logits, lengths0, dims, B, TD, L, torch, np)
    fp8x = {}
    if not args.no_fp8_cross:
        ckv = torch.empty(Ldec, 2, B, H, T, 64, dtype=torch.bfloat16, device=DEV)
        for fmt in (None, "e4m3", "e5m2"):
            fp8x[fmt] = cross_kv_step(model, audio, mel, enc, ckv, state, tokens, logits, lengths0, dims, B, TD, L,
                                      torch, np, DecodeState, fmt)
        del ckv
        torch.cuda.empty_cache()

    kernels = {}
    if not args.no_kernel_probes:
        kernels = kernel_probes(model, mel, enc, state, tokens, logits, lengths0, dims, B, TD, L, torch, np)
        # decode attention of one layer as a whole (the cross-attention over the
        # encoder output timed in the timed region, the self-attention over the
        # fp8 cache by its probe; bytes at each measurement's own lengths)
        sa = kernels["decode_self_attention_fp8"]
        by = cross_bytes + sa["bytes_per_launch"]
        us = cross_ms * 1e3 + sa["avg_launch_us"]
        kernels["decode_attention_per_layer"] = {
            "bound": "hbm", "achieved": round(by / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes": round(by), "us": round(us, 2),
            "parts": "attn_cross_enc_kernel (timed region) + attn_decode_self_kernel (probe)"}

    result = {
        "metric": "RTFx and decode tok/s at Whisper large-v3 shape, fp8 KV, batch 64",
        "value": round(rtfx, 2),
        "unit": "x realtime (audio s / wall s)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded tones + noise audio, random N(0,0.02) weights, seeded token ids)",
        "config": {"workload": f"large-v3 full path: {B} x 30 s chunks -> log-mel -> 32-layer encoder -> "
                               f"{TD} teacher-forced decode steps, batch {B}, fp8 e4m3 self-KV "
                               f"prefilled U[1,448], cap {cap}; cross-attention over the encoder output "
                               f"in absorbed form",
                   "batch": B, "decode_steps": TD, "audio_s_per_step": B * AUDIO_S},
        "decode_tok_per_s": round(decode_tok_s, 1),
        "encoder_tflops": round(enc_flop / (stage_ms["encode"] * 1e-3) / 1e12, 1),
        "stage_ms": {k: round(v, 3) for k, v in stage_ms.items()},
        "roofline": {"kernel": "attn_cross_enc_kernel (decoder cross-attention over the encoder output)",
                     "bound": "hbm", "achieved": round(cross_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(cross_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic("attn_cross_enc_kernel"),
                     "bytes_per_launch": cross_bytes, "avg_launch_us": round(cross_ms * 1e3, 2),
                     "launches_timed": n_rec},
        "kernels": kernels,
    }
    if peaks is not None:
        result["measured_peaks"] = peaks
        rl = result["roofline"]
        rl["peak_measured"], rl["frac_of_measured"] = peaks["hbm_read_gbs"], round(cross_gbs / peaks["hbm_read_gbs"], 4)
        for k in kernels.values():
            ref = peaks["hbm_read_gbs"] if k["bound"] == "hbm" else peaks["mfma_bf16_tflops"]
            k["peak_measured"], k["frac_of_measured"] = ref, round(k["achieved"] / ref, 4)
    if lf is not None:
        result["long_form"] = lf
    if fp8e is not None:
        if peaks is not None:
            k = fp8e["encoder_ffn1_gemm_fp8"]
            k["peak_measured_bf16"] = peaks["mfma_bf16_tflops"]
        result["mixed_fp8"] = fp8e
    for fmt, leg in fp8x.items():
        if peaks is not None:
            xc = leg["cross_attention"]
            xc["peak_measured"] = peaks["hbm_read_gbs"]
            xc["frac_of_measured"] = round(xc["achieved"] / peaks["hbm_read_gbs"], 4)
        result[{None: "bf16_cross_kv", "e4m3": "fp8_cross_kv", "e5m2": "fp8_cross_kv_e5m2"}[fmt]] = leg
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(dims, audio, lengths0, tokens, state, np, torch, prefill_max)
    print(json.dumps(result))


def kernel_probes(model, mel, enc, state, tokens, logits, lengths0, dims, B, TD, L, torch, np):
    """Per-kernel rooflines of the other hot kernels, each timed with the same
    event hook in one extra (untimed) pass of the stage that launches it."""
    out = {}
    d, T, F, H = dims.d_model, dims.n_audio_ctx, dims.d_ffn, dims.n_heads
    M = B * T

    def timed(kind, fn, cap):
        s = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
        for x in s + e:
            x.record()
        torch.cuda.synchronize()
        L.whisper_profile_arm(kind, s, e)
        fn()
        torch.cuda.synchronize()
        n = L.whisper_profile_disarm()
        return float(np.mean([s[i].elapsed_time(e[i]) for i in range(n)])), n

    ms, n = timed(L.PROF_ENCODER_FFN1, lambda: model.encode(mel, out=enc), 32)
    fl = 2.0 * M * d * F
    out["encoder_ffn1_gemm"] = {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                "avg_launch_us": round(ms * 1e3, 1), "launches": n,
                                "shape": f"[{M},{d}]x[{d},{F}] + bias + GELU"}
    ms, n = timed(L.PROF_ENCODER_ATTENTION, lambda: model.encode(mel, out=enc), 32)
    fl = 4.0 * B * H * T * T * 64
    out["encoder_attention"] = {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 1),
                                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                "avg_launch_us": round(ms * 1e3, 1), "launches": n}
    ms, n = timed(L.PROF_ENCODER_LAYERNORM, lambda: model.encode(mel, out=enc), 32)
    by = M * d * (2 + 4 + 4 + 2)
    out["encoder_residual_layernorm"] = {"bound": "hbm", "achieved": round(by / (ms * 1e-3) / 1e9, 1),
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                         "avg_launch_us": round(ms * 1e3, 1), "launches": n,
                                         "bytes_per_launch": by}
    n_steps = 8

    def dec():
        state.lengths.copy_(lengths0)
        for t in range(n_steps):
            model.decode_step(state, tokens[t], logits)

    mean_len = float(lengths0.float().mean().item()) + (n_steps - 1) / 2 + 1
    ms, n = timed(L.PROF_DECODE_SELF_ATTENTION, dec, dims.n_dec_layers * n_steps)
    by = 2 * B * H * mean_len * 64 + B * d * 4
    out["decode_self_attention_fp8"] = {"bound": "hbm", "achieved": round(by / (ms * 1e-3) / 1e9, 1),
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "avg_launch_us": round(ms * 1e3, 1), "launches": n,
                                        "bytes_per_launch": round(by)}
    return out


def long_form(L, torch, Whisper, DecodeState):
    """The pages' long-form workload, end to end: 45 min of 16 kHz synthetic
    audio (piecewise 2-8 s tone / noise segments) as 90 x 30 s chunks -> GPU
    log-mel -> 32-layer encoder -> 4 prompt + 224 teacher-forced decode steps
    of the 4 decoder layers at batch 90 (cross-attention over the encoder
    output), fp8 KV cache from empty (cap 228; the prompt fed by one causal
    prefill), at the large-v3-turbo shape with random weights. One
    warm-up pass, then one timed pass; RTFx = 2700 s of audio / wall time."""
    from workload import CONFIGS, gen_audio_longform, gen_tokens, gen_weights
    from workload.configs import RUN
    dims = CONFIGS["turbo_longform"]
    run = RUN["turbo_longform"]
    B, n_tok, cap = run["batch"], run["prompt"] + run["steps"], run["cap"]
    W = gen_weights("cuda", dims)
    m = Whisper(dims, list(W.values()))
    del W
    torch.cuda.empty_cache()
    audio = gen_audio_longform("cuda", dims.cfg_id, run["minutes"])
    assert audio.shape[0] == B
    tokens = gen_tokens("cuda", dims.cfg_id, n_tok, B, dims.n_vocab)
    mel = torch.empty(B, dims.n_mels, 3000, dtype=torch.float32, device="cuda")
    enc = torch.empty(B, dims.n_audio_ctx, dims.d_model, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(B, dims.n_vocab, dtype=torch.float32, device="cuda")
    state = DecodeState(dims, B, cap, None, torch.ones(dims.n_dec_layers, 2), torch.zeros(B, dtype=torch.int32),
                        enc=enc)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    prompt = tokens[:run["prompt"]].t().contiguous()

    def once(record):
        if record: ev[0].record()
        m.logmel(audio, out=mel)
        if record: ev[1].record()
        m.encode(mel, out=enc)
        if record: ev[2].record()
        state.lengths.zero_()
        m.decode_prefill(state, prompt, logits)   # the prompt tokens in one causal pass
        if record: ev[3].record()
        for t in range(run["prompt"], n_tok):
            m.decode_step(state, tokens[t], logits)
        if record: ev[4].record()

    once(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    once(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(state.dev_error[0].item()) == 0
    audio_s = run["minutes"] * 60.0
    # host to host: the audio starts in pinned host memory and every decoded
    # token id ends on the host (the upload, the per-step id copies and the
    # download are inside the timed region)
    audio_host = audio.cpu().pin_memory()
    ids = torch.empty(n_tok, B, dtype=torch.int32, device="cuda")
    ids_host = torch.empty(n_tok, B, dtype=torch.int32).pin_memory()

    def host_to_host():
        audio.copy_(audio_host, non_blocking=True)
        m.logmel(audio, out=mel)
        m.encode(mel, out=enc)
        state.lengths.zero_()
        ids[run["prompt"] - 1].copy_(m.decode_prefill(state, prompt, logits))
        for t in range(run["prompt"], n_tok):
            ids[t].copy_(m.decode_step(state, tokens[t], logits))
        ids_host.copy_(ids, non_blocking=True)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host_to_host()
    torch.cuda.synchronize()
    wall_h2h = time.perf_counter() - t0
    assert int(state.dev_error[0].item()) == 0
    st = {n: round(ev[i].elapsed_time(ev[i + 1]), 3)
          for i, n in enumerate(["logmel", "encode", "prefill", "decode"])}
    log(f"long form: {audio_s:.0f} s of audio in {wall * 1e3:.1f} ms, RTFx {audio_s / wall:.0f}, stages {st}; "
        f"host to host {wall_h2h * 1e3:.1f} ms, RTFx {audio_s / wall_h2h:.0f}")
    out = {"workload": f"large-v3-turbo shape (32 encoder, 4 decoder layers): {run['minutes']:.0f} min of 16 kHz "
                       f"synthetic audio -> {B} x 30 s chunks -> log-mel -> encoder -> "
                       f"{run['prompt']} prompt tokens in one causal prefill + {run['steps']} teacher-forced "
                       f"decode steps (cross-attention over the encoder output), batch {B}, "
                       f"fp8 e4m3 self-KV from empty, cap {cap}",
           "rtfx": round(audio_s / wall, 1), "ms": round(wall * 1e3, 3), "stage_ms": st,
           "rtfx_host_to_host": round(audio_s / wall_h2h, 1),
           "host_to_host": "fp32 audio uploaded from pinned host memory, the token ids of every step copied "
                           "out and downloaded, inside the timed region",
           "decode_tok_per_s": round(B * run["steps"] / (st["decode"] * 1e-3), 1),
           "data": "synthetic (seeded piecewise tone/noise audio, random N(0,0.02) weights, seeded token ids)"}
    del m, audio, mel, enc, logits, state, audio_host, ids, ids_host
    torch.cuda.empty_cache()
    return out


def measured_peaks(L, torch):
    """The rates this part sustains: bf16 MFMA with register-resident operands
    (16,384 waves, 16 independent accumulator chains each) and a streaming read
    of a 4 GiB buffer (16 times the last-level cache). Best of 3 timed runs
    after a warm-up."""
    n_wg, iters = 4096, 1000
    out = torch.empty(n_wg * 4, device="cuda")
    L.whisper_peak_mfma(n_wg, 20, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        e0.record(); L.whisper_peak_mfma(n_wg, iters, out); e1.record(); torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    mfma = L.whisper_peak_mfma_flop(n_wg, iters) / (best * 1e-3) / 1e12
    nbytes, n_wg_r = 4 << 30, 8192
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outr = torch.empty(n_wg_r, device="cuda")
    L.whisper_peak_read(buf, nbytes, n_wg_r, outr)
    best = float("inf")
    for _ in range(3):
        e0.record(); L.whisper_peak_read(buf, nbytes, n_wg_r, outr); e1.record(); torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del buf
    torch.cuda.empty_cache()
    read = nbytes / (best * 1e-3) / 1e9
    log(f"measured peaks: bf16 MFMA {mfma:.0f} TFLOP/s, HBM read {read:.0f} GB/s")
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_gbs": round(read, 1),
            "how": "register-resident MFMA 16x16x32 bf16 loop, 16384 waves; 16-byte streaming read of 4 GiB"}


def fp8_encoder_step(model, audio, mel, enc, state, tokens, logits, lengths0, dims, B, TD, L, torch, np):
    """One more full step with the mixed_fp8 preset's sites in E4M3: the
    encoder's query, key, value, fc1, fc2 (per-tensor weight and per-chunk
    activation amax scales) and the decoder MLP's fc1, fc2 (per-tensor weight
    and per-token activation scales), the rest unchanged. Reported apart from
    `value`: the configured workload is bf16."""
    def step(ev=None):
        if ev: ev[0].record()
        model.logmel(audio, out=mel)
        model.encode_fp8(mel, out=enc)
        if ev: ev[1].record()
        state.lengths.copy_(lengths0)
        for t in range(TD):
            model.decode_step(state, tokens[t], logits)
        if ev: ev[2].record()

    state.ffn_fp8 = True
    try:
        step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t0 = time.perf_counter()
        step(ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        state.ffn_fp8 = False
    assert int(state.dev_error[0].item()) == 0
    # the fc1 site (E4M3 GEMM + bias + GELU) with the event hook, in one more encoder pass
    n = 32
    s = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    e = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for x in s + e:
        x.record()
    torch.cuda.synchronize()
    L.whisper_profile_arm(L.PROF_ENCODER_FFN1, s, e)
    t1 = time.perf_counter()
    model.encode_fp8(mel, out=enc)
    torch.cuda.synchronize()
    enc_wall = time.perf_counter() - t1
    n_rec = L.whisper_profile_disarm()
    ms = float(np.mean([s[i].elapsed_time(e[i]) for i in range(n_rec)]))
    M, d, F = B * dims.n_audio_ctx, dims.d_model, dims.d_ffn
    fl = 2.0 * M * d * F
    tf = fl / (ms * 1e-3) / 1e12
    log(f"mixed_fp8 step: {wall * 1e3:.1f} ms, encode {ev[0].elapsed_time(ev[1]):.1f} ms, decode "
        f"{ev[1].elapsed_time(ev[2]):.1f} ms, encoder fc1 fp8 GEMM {ms * 1e3:.0f} us ({tf:.0f} TFLOP/s)")
    return {"ms_per_step": round(wall * 1e3, 3), "rtfx": round(B * AUDIO_S / wall, 2),
            "stage_ms": {"logmel_encode": round(ev[0].elapsed_time(ev[1]), 3),
                         "decode": round(ev[1].elapsed_time(ev[2]), 3)},
            "encode_only_ms": round(enc_wall * 1e3, 3),
            "encoder_ffn1_gemm_fp8": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(tf / FP8_PEAK_TFLOPS, 4),
                                      "avg_launch_us": round(ms * 1e3, 1), "launches": n_rec,
                                      "shape": f"[{M},{d}]x[{d},{F}] E4M3 + scales + bias + GELU"},
            "note": "mixed_fp8 preset sites in E4M3 (encoder query/key/value, fc1, fc2; decoder fc1, fc2); "
                    "not the configured workload"}


def cross_kv_step(model, audio, mel, enc, ckv, state, tokens, logits, lengths0, dims, B, TD, L, torch, np,
                  DecodeState, fmt=None):
    """One more full step through explicit cross-attention K/V: the K/V of
    every decoder layer projected once per batch (whisper_cross_kv), then the
    decode reads them, as bf16 (fmt None, whisper_decode_step) or as fp8 codes
    in `fmt` ("e4m3", or "e5m2" as the aggressive preset has it; one amax
    scale per layer and K|V, quantised inside the step; whisper_decode_step_xq).
    Reported apart from `value`: the configured workload reads the encoder
    output in absorbed form instead."""
    H, T = dims.n_heads, dims.n_audio_ctx
    code = None if fmt is None else {"e4m3": L.WHISPER_FP8_E4M3, "e5m2": L.WHISPER_FP8_E5M2}[fmt]
    xcodes = None if fmt is None else torch.empty(ckv.shape, dtype=torch.uint8, device=ckv.device)
    sx = DecodeState(dims, 1, 1, None if fmt else ckv, state.kv_scales, lengths0[:1],
                     cross_format=code if fmt else L.WHISPER_FP8_E4M3)  # small placeholder cache, replaced below
    sx.batch, sx.cap, sx.kv_cache, sx.lengths = B, state.cap, state.kv_cache, state.lengths
    sx.argmax, sx.dev_error = state.argmax, state.dev_error

    def step(ev=None):
        if ev: ev[0].record()
        model.logmel(audio, out=mel)
        model.encode(mel, out=enc)
        model.cross_kv(enc, out=ckv)
        if ev: ev[1].record()
        if fmt is not None:
            sx.cross_codes, sx.cross_scales = model.quantize_cross_kv(ckv, codes=xcodes, fmt=code)
        if ev: ev[2].record()
        state.lengths.copy_(lengths0)
        for t in range(TD):
            model.decode_step(sx, tokens[t], logits)
        if ev: ev[3].record()

    step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    n_ev = min(2048, dims.n_dec_layers * TD)
    ks = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ke = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in ks + ke:
        e.record()
    torch.cuda.synchronize()
    L.whisper_profile_arm(L.PROF_DECODE_CROSS_ATTENTION, ks, ke)
    t0 = time.perf_counter()
    step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_rec = L.whisper_profile_disarm()
    assert int(state.dev_error[0].item()) == 0
    x_ms = float(np.mean([ks[i].elapsed_time(ke[i]) for i in range(n_rec)]))
    elt = 2 if fmt is None else 1
    x_bytes = 2 * B * H * T * 64 * elt + 2 * B * dims.d_model * 2  # K and V, q in, output out
    dec_ms = ev[2].elapsed_time(ev[3])
    name = fmt or "bf16"
    log(f"{name} cross K/V step: {wall * 1e3:.1f} ms, decode {dec_ms:.1f} ms, cross-attention {x_ms * 1e3:.1f} us "
        f"({x_bytes / (x_ms * 1e-3) / 1e9:.0f} GB/s)")
    stage = {"logmel_encode_cross_kv": round(ev[0].elapsed_time(ev[1]), 3), "decode": round(dec_ms, 3)}
    if fmt is not None:
        stage["quantize_cross_kv"] = round(ev[1].elapsed_time(ev[2]), 3)
    return {"ms_per_step": round(wall * 1e3, 3), "rtfx": round(B * AUDIO_S / wall, 2),
            "decode_tok_per_s": round(B * TD / (dec_ms * 1e-3), 1), "stage_ms": stage,
            "cross_attention": {"bound": "hbm", "bytes_per_launch": x_bytes, "avg_launch_us": round(x_ms * 1e3, 2),
                                "achieved": round(x_bytes / (x_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(x_bytes / (x_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "launches_timed": n_rec},
            "note": (f"{fmt} cross-attention K/V, one amax scale per layer and K|V" if fmt else
                     "bf16 cross-attention K/V projected once per batch") + "; not the configured workload"}


def cpu_baseline(dims, audio, lengths0, tokens, state, np, torch, prefill_max):
    """The oracle, untouched, on a bounded sample of the same workload: chunk 0
    through log-mel, the 32-layer encoder and cross K/V, then N_DEC of its 224
    decode steps (batch 1); decode time is scaled to 224 steps."""
    import importlib
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    O = importlib.import_module("oracle.whisper_oracle")
    from workload import gen_prefill_kv, gen_weights
    N_DEC = 8
    W = {k: v.double().cpu().numpy() for k, v in gen_weights("cuda", dims).items()}
    H, Ld = dims.n_heads, dims.n_dec_layers
    a0 = audio[0].cpu().numpy()
    t = time.perf_counter()
    m = O.log_mel(a0, dims.n_mels)
    e = O.encoder(m, W, H, dims.n_enc_layers)
    cr = O.cross_kv(e, W, H, Ld)
    t_front = time.perf_counter() - t
    cross = [({0: k}, {0: v}) for k, v in cr]
    # row 0's prefilled cache from the seeded prefill values, through the
    # oracle's own scale and codec
    cap = state.kv_cache.shape[4]
    cache = [[{0: np.zeros((H, cap, 64), np.uint8)} for kv in range(2)] for l in range(Ld)]
    sc = np.ones((Ld, 2), np.float32)
    for l in range(Ld):
        for kv in range(2):
            x = gen_prefill_kv("cuda", dims.cfg_id, l, kv, audio.shape[0], H, prefill_max)
            sc[l, kv] = O.e4m3_scale_from_amax(np.array([x.abs().max().item()], np.float32))
            cache[l][kv][0][:, :prefill_max] = O.e4m3_quantize(x[0].cpu().numpy(), sc[l, kv])
            del x
    tok = tokens.cpu().numpy()
    length = np.array([int(lengths0[0].item())])
    t = time.perf_counter()
    for s in range(N_DEC):
        O.decode_step(W, H, tok[s, :1], length, cache, sc, cross)
        length = length + 1
    t_dec = (time.perf_counter() - t) * (tokens.shape[0] / N_DEC)
    total = t_front + t_dec
    return {"value": round(AUDIO_S / total, 3), "unit": "x realtime (audio s / wall s)", "cores": int(cores),
            "kind": "oracle", "dtype": "f64",
            "sample": f"chunk 0 of the batch: log-mel + 32-layer encoder + cross K/V ({t_front:.1f} s) and "
                      f"{N_DEC} of {tokens.shape[0]} decode steps at batch 1, scaled x{tokens.shape[0] / N_DEC:.0f} "
                      f"({t_dec:.1f} s); fp64 NumPy"}


if __name__ == "__main__":
    main()
