"""Throughput of one Wan2.1 CFG denoise step on one MI355X.

One step = the whole hot path on the 1.3B 480p x 81-frame workload: patchify,
time modulation, 30 DiT blocks over the CFG batch of two (cond + null text
context), the head, guidance and the Euler update (wan_denoise_step).  Inputs
and weights are seeded synthetic tensors of the real shapes, resident in HBM
before the timed region.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config wan13b_step] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from video_diffusion_transformer_forward_amd import synth as S  # noqa: E402

MI355X_BF16_TFLOPS = 2516.6   # dense bf16 MFMA peak (256 CU x 4096 flop/clk x 2.4 GHz)
MI355X_FP32_TFLOPS = 157.3
CALIB_COPY_BYTES = 1 << 30   # bytes read (and written) by the calibration copy

# L2 <-> memory bytes of one self-attention launch (the static-offset kernel plus its flagged-workgroup
# pass), from two counter-collection runs of
# `bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-cache-modes --no-vae --no-qk8 --block-configs "" --calib-copy`
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, means over the launches of each kernel, summed), each
# scaled by known/counted bytes of the 1 GiB calibration copy in the same run.  Valid only for the kernel
# sources they were taken on (checked by hash; later comment and static_assert edits were re-hashed after checking that the
# generated device code is unchanged).
ATTN_COUNTERS = {
    "fetch_kib": 885137.94 + 117.01, "fetch_scale": 1048576 / 524302.67,
    "write_kib": 196656.0 + 0.0, "write_scale": 1048576 / 1048576.0,
    "sources": ("video_diffusion_transformer_forward_amd/csrc/attention.hip",
                "video_diffusion_transformer_forward_amd/csrc/common.h"),
    "sha256": "7f8899957fe59dc0507d84bb809b526b266f2f2fd8da38a75f00fecdf42fbb13",
}

METRIC = "DiT block TFLOP/s (%bf16 MFMA peak) + ms/denoise step, 1.3B @ 480p×81f"


def block_flops(cfg: S.WanConfig, batch: int) -> dict:
    """Algorithmic FLOPs of one block over `batch` videos: 2MNK per GEMM, 4 Lq Lk D per attention."""
    L, D, F, Lt, Li = cfg.seq_len, cfg.dim, cfg.ffn_dim, cfg.txt_len, cfg.img_len
    M = batch * L
    f = {
        "qkv": 2 * M * D * 3 * D,
        "self_attention": 4 * batch * L * L * D,
        "o_proj": 2 * M * D * D,
        "cross_q": 2 * M * D * D,
        "ctx_kv": 2 * batch * (Lt + Li) * D * 2 * D,
        "cross_attention": 4 * batch * L * (Lt + Li) * D,
        "cross_o": 2 * M * D * D,
        "ffn1": 2 * M * D * F,
        "ffn2": 2 * M * F * D,
    }
    return f


def step_flops(cfg: S.WanConfig) -> float:
    B2 = 2 * cfg.batch
    M = B2 * cfg.seq_len
    per_block = sum(block_flops(cfg, B2).values())
    patch = 2 * M * cfg.patch_k * cfg.dim
    head = 2 * M * cfg.dim * 64
    time_mlp = 2 * (256 * cfg.dim + cfg.dim * cfg.dim + 6 * cfg.dim * cfg.dim)
    return cfg.n_blocks * per_block + patch + head + time_mlp


class ClockSampler:
    """Samples the current GPU core and memory clock levels (sysfs pp_dpm_sclk / pp_dpm_mclk, the
    line marked '*') every `period` seconds on a background thread; reads only."""

    def __init__(self, period: float = 0.25):
        import glob
        import threading
        self.files = {}
        for kind in ("sclk", "mclk"):
            found = sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}"))
            if found:
                self.files[kind] = found[0]
        self.samples = {k: [] for k in self.files}
        self.period = period
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, path):
        try:
            with open(path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, f in self.files.items():
                v = self._read(f)
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.files:
            self._thread.join(timeout=2.0)

    def summary(self):
        out = {}
        for k, v in self.samples.items():
            if v:
                v = sorted(v)
                out[f"{k}_mhz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1], "samples": len(v)}
        return out or None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_block(bcfg: S.WanConfig, reps: int = 6, n_sets: int = 3) -> dict:
    """ms and TFLOP/s of one wan_dit_block_forward on a single video of bcfg's shape (inputs resident).
    The timed calls rotate over n_sets distinct weight sets, so that one block's weights (93 MB at the
    1.3B shape) are not served from the 256 MB Infinity Cache every time."""
    import torch
    import video_diffusion_transformer_forward_amd as W
    from video_diffusion_transformer_forward_amd import _native as N
    blks = [W.DeviceBlock(bcfg, S.block_weights(bcfg, b)) for b in range(n_sets)]
    x = torch.from_numpy(S.block_inputs(bcfg)).cuda()
    mod = torch.from_numpy(S.modulation(bcfg)).cuda()
    ctx = torch.from_numpy(S.context(bcfg, "cond")).to(W.elem_dtype(bcfg)).cuda()
    ws = W.workspace(bcfg, N.ENTRY_BLOCK)
    for b in range(n_sets):
        W.dit_block_forward(bcfg, blks[b], x, mod, ctx, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(reps):
        W.dit_block_forward(bcfg, blks[i % n_sets], x, mod, ctx, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    fl = sum(block_flops(bcfg, bcfg.batch).values())
    del blks, x, mod, ctx, ws
    torch.cuda.empty_cache()
    return {"ms_per_block": round(ms, 3), "block_tflop": round(fl / 1e12, 3),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "seq_len": bcfg.seq_len, "dim": bcfg.dim,
            "weight_sets": n_sets}


def vae_flops(vcfg) -> float:
    """Algorithmic FLOPs of one whole-video decode: 2 x voxels x C_out x (taps x C_in) per convolution."""
    from video_diffusion_transformer_forward_amd import vae_synth as VS
    T, H, W = vcfg.frames, vcfg.height, vcfg.width
    frames = [T, 2 * T - 1, 4 * T - 3, 4 * T - 3]   # per level: latent, after each time doubling
    total = 0.0
    for name, shape in VS.vae_param_shapes(vcfg):
        if len(shape) != 5:
            continue
        cout, kt, kh, kw, cin = shape
        if name == "conv_in" or name.startswith("mid."):
            lvl = 0
        elif name.startswith("head."):
            lvl = 3
        else:
            s = int(name.split(".")[1])
            lvl = s + 1 if name.endswith("space_conv") else s
        nf = frames[lvl]
        if name.endswith("time_conv"):
            nf = frames[lvl] - 1          # the first frame passes through
        vox = nf * (H << lvl) * (W << lvl)
        total += 2.0 * vox * cout * kt * kh * kw * cin
    return total


def time_vendor_gemms(cfg: S.WanConfig, reps: int = 10) -> dict:
    """The step's projections through torch.nn.functional.linear (hipBLASLt) on the same shapes (CFG batch 2,
    M = 2L rows), alone and followed by the work this library's GEMM epilogues fuse, done as separate torch
    passes: GELU (erf) after FFN1; the gated float32 residual x += g * y after FFN2 and the output projections;
    RoPE on q and k and the head-major q / k / transposed-v layout after QKV.  Random bf16 operands; ms per
    launch, timed with events on torch's stream.  A measurement of the vendor library, not a path of this
    library."""
    import torch
    import torch.nn.functional as F
    dev, bf = "cuda", torch.bfloat16
    L, D, Fd, H = cfg.seq_len, cfg.dim, cfg.ffn_dim, cfg.heads
    hd, M = D // H, 2 * cfg.seq_len
    g = torch.Generator(device=dev).manual_seed(7)

    def rnd(*shape, dtype=bf, scale=0.02):
        return (torch.randn(*shape, device=dev, generator=g, dtype=torch.float32) * scale).to(dtype)

    m, hbuf = rnd(M, D, scale=1.0), rnd(M, Fd, scale=0.1)
    x = rnd(M, D, dtype=torch.float32, scale=1.0)
    gate = rnd(D, dtype=torch.float32, scale=0.1)
    w = {"qkv": rnd(3 * D, D), "o": rnd(D, D), "ffn1": rnd(Fd, D), "ffn2": rnd(D, Fd)}
    b = {k: rnd(v.shape[0]) for k, v in w.items()}
    ang = torch.rand(L, hd // 2, device=dev, generator=g) * 6.28
    cos, sin = torch.cos(ang).to(bf), torch.sin(ang).to(bf)

    def rope(t):  # (2, L, H, hd) -> rotated adjacent pairs
        t2 = t.view(2, L, H, hd // 2, 2)
        c, s_ = cos.view(1, L, 1, hd // 2), sin.view(1, L, 1, hd // 2)
        return torch.stack((t2[..., 0] * c - t2[..., 1] * s_, t2[..., 0] * s_ + t2[..., 1] * c), -1).view(2, L, H, hd)

    def qkv_epi(y):
        y = y.view(2, L, 3, H, hd)
        q = rope(y[:, :, 0]).permute(0, 2, 1, 3).contiguous()
        k = rope(y[:, :, 1]).permute(0, 2, 1, 3).contiguous()
        vt = y[:, :, 2].permute(0, 2, 3, 1).contiguous()
        return q, k, vt

    cases = {
        "qkv": (lambda: F.linear(m, w["qkv"], b["qkv"]), qkv_epi, 2 * M * D * 3 * D),
        "o_proj": (lambda: F.linear(m, w["o"], b["o"]), lambda y: x.addcmul_(gate, y), 2 * M * D * D),
        "ffn1": (lambda: F.linear(m, w["ffn1"], b["ffn1"]), lambda y: F.gelu(y), 2 * M * D * Fd),
        "ffn2": (lambda: F.linear(hbuf, w["ffn2"], b["ffn2"]), lambda y: x.addcmul_(gate, y), 2 * M * Fd * D),
    }
    out = {}
    for name, (gemm, epi, flop) in cases.items():
        res = {}
        for label, fn in (("gemm_ms", gemm), ("gemm_plus_epilogue_ms", lambda: epi(gemm()))):
            for _ in range(2):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(reps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            res[label] = round(ev[0].elapsed_time(ev[1]) / reps, 4)
        res["gemm_tflops"] = round(flop / (res["gemm_ms"] * 1e-3) / 1e12, 1)
        out[name] = res
    del m, hbuf, x, w
    torch.cuda.empty_cache()
    return out


def time_vae(name: str = "vae_480p", reps: int = 3) -> dict:
    """Whole-video decode of the 81-frame 480p latent (one call), timed with torch events."""
    import torch
    import video_diffusion_transformer_forward_amd as W
    from video_diffusion_transformer_forward_amd import vae_synth as VS
    vcfg = VS.get_vae_config(name)
    sh = W.vae_shape_of(vcfg)
    dev = W.VaeDevice(sh, VS.vae_params(vcfg))
    ws = W.vae_workspace(sh)
    cache = W.vae_cache(sh)
    z = torch.from_numpy(VS.vae_latent(vcfg)).cuda()
    video = torch.empty((3, vcfg.out_frames, vcfg.out_height, vcfg.out_width), dtype=torch.float32, device="cuda")
    W.vae_decode(sh, dev, z, 0, vcfg.frames, cache, video, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        W.vae_decode(sh, dev, z, 0, vcfg.frames, cache, video, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    assert bool(torch.isfinite(video).all())
    fl = vae_flops(vcfg)
    out = {"workload": f"{name}: latent 16x{vcfg.frames}x{vcfg.height}x{vcfg.width} -> video 3x{vcfg.out_frames}x"
                       f"{vcfg.out_height}x{vcfg.out_width}, widths {list(vcfg.dims)}, {vcfg.n_res} residual blocks "
                       f"per stage, one call",
           "ms_per_video": round(ms, 2), "tflop": round(fl / 1e12, 2),
           "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
           "workspace_gb": round(ws.numel() / 1e9, 2)}
    del ws, cache, video, dev
    torch.cuda.empty_cache()
    return out


def time_stream(cfg, model, ctx, slots: int = 4, group: int = 1, ticks: int = 10) -> dict:
    """Streaming queue at the 1.3B 480p shape: a window of `slots` x `group` latent frames
    (60 x 104), one tick = one guidance-free DiT pass over the window + the queue update, then
    the emitted latent frames decoded by the VAE through its feature cache (4 video frames each)."""
    import torch
    import numpy as np
    import video_diffusion_transformer_forward_amd as W
    from video_diffusion_transformer_forward_amd import vae_synth as VS
    scfg = cfg.with_(frames=slots * group, batch=1)
    taus = [1000.0 * (1.0 - (slots - 1 - k) / slots) for k in range(slots)]
    dts = [1.0 / slots] * slots
    ws = W.stream_workspace(scfg, group)
    win = torch.from_numpy(S.latent(scfg)).cuda()
    noise = torch.from_numpy(np.random.default_rng(0).standard_normal(
        (1, 16, group, scfg.height, scfg.width)).astype(np.float32)).cuda()
    out = torch.empty_like(noise)
    vcfg = VS.get_vae_config("vae_480p")
    vsh = W.vae_shape_of(vcfg, group)
    vdev = W.VaeDevice(vsh, VS.vae_params(vcfg))
    vws = W.vae_workspace(vsh)
    vcache = W.vae_cache(vsh)
    video = torch.empty((3, 4 * group, vcfg.out_height, vcfg.out_width), dtype=torch.float32, device="cuda")
    first = torch.empty((3, 4 * group - 3, vcfg.out_height, vcfg.out_width), dtype=torch.float32, device="cuda")

    def tick(i, decode):
        W.stream_tick(scfg, model, win, ctx, taus, dts, group, noise, out, ws)
        if decode:
            t0 = i * group
            W.vae_decode(vsh, vdev, out[0], t0, group, vcache, first if t0 == 0 else video, vws)

    tick(0, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(1, ticks + 1):
        tick(i, False)
    torch.cuda.synchronize()
    ms_tick = (time.perf_counter() - t1) / ticks * 1e3
    t1 = time.perf_counter()
    for i in range(1, ticks + 1):
        tick(i, True)
    torch.cuda.synchronize()
    ms_both = (time.perf_counter() - t1) / ticks * 1e3
    assert bool(torch.isfinite(win).all()) and bool(torch.isfinite(video).all())
    del ws, vws, vcache
    torch.cuda.empty_cache()
    return {"workload": f"1.3B DiT, window of {slots} slots x {group} latent frame(s) at 60x104 "
                        f"(L={slots * group * 1560}), one guidance-free pass per tick; VAE decode of the emitted "
                        f"frame(s) through the feature cache",
            "ms_per_tick_dit": round(ms_tick, 2), "ms_per_tick_with_vae": round(ms_both, 2),
            "video_frames_per_tick": 4 * group,
            "video_fps": round(4 * group / (ms_both * 1e-3), 1)}


def attn_traffic_bytes():
    """Counted bytes per self-attention launch, or None once its sources differ from the measured ones."""
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_COUNTERS["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != ATTN_COUNTERS["sha256"]:
        return None
    c = ATTN_COUNTERS
    return round(c["fetch_kib"] * 1024 * c["fetch_scale"] + c["write_kib"] * 1024 * c["write_scale"])


def cpu_baseline(cfg: S.WanConfig, budget_s: float = 20.0) -> dict:
    """The float64 oracle on a bounded sample of the same workload: one 1.3B block with the
    keys/values of all 32760 tokens and the outputs of a sample of query rows."""
    from oracle import wan_oracle as O
    bcfg = cfg.with_(n_blocks=1)
    w = S.block_weights(bcfg, 0)
    x = S.block_inputs(bcfg)
    mod = S.modulation(bcfg)
    ctx = S.context(bcfg, "cond")
    L, D, F = bcfg.seq_len, bcfg.dim, bcfg.ffn_dim
    n_rows = 8192
    rows = np.linspace(0, L - 1, n_rows).astype(int).tolist()
    t0 = time.perf_counter()
    O.dit_block(x, mod, ctx, w, bcfg.heads, bcfg.grid, bcfg.img_len, rows=rows)
    dt = time.perf_counter() - t0
    # algorithmic FLOPs actually performed by the sample
    n = len(rows)
    fl = (2 * L * D * 2 * D                      # k, v projections of every token
          + 2 * n * D * D                        # q of the sampled rows
          + 4 * n * L * D                        # self-attention of the sampled rows
          + 2 * n * D * D * 3                    # o, cross q, cross o
          + 2 * bcfg.txt_len * D * 2 * D         # context k, v
          + 4 * n * bcfg.txt_len * D             # cross-attention
          + 4 * n * D * F)                       # FFN
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"float64 oracle, one 1.3B block (L=32760, D=1536): k/v of all tokens, outputs of {n} "
                      f"query rows; {fl / 1e12:.3f} TFLOP in {dt:.1f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="wan13b_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-modes", action="store_true", help="skip timing the diffusion-cache step modes")
    ap.add_argument("--no-qk8", action="store_true", help="skip timing the step in the 8-bit forms")
    ap.add_argument("--no-vae", action="store_true", help="skip timing the 480p x 81-frame VAE decode")
    ap.add_argument("--no-graph", action="store_true", help="skip timing the step replayed from a HIP graph")
    ap.add_argument("--vendor-gemms", action="store_true",
                    help="also time the step's projections through hipBLASLt (torch), alone and with their "
                         "epilogue work as separate passes (reported under 'vendor_gemms')")
    ap.add_argument("--vae-only", action="store_true",
                    help="time only the VAE decode and print its JSON object (for profiling runs)")
    ap.add_argument("--block-configs", default="wan13b_block,wan14b_720p_block,wan14b_i2v_block",
                    help="comma-separated block configurations to time one block forward of (a single "
                         "video, rotating over 3 weight sets); reported under 'blocks'; '' skips them")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB -> 1 GiB elementwise copy three times: the "
                         "known-size kernel that scales the HBM byte counters of a counter-collection run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the hot path here is one GPU's share of the work "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import video_diffusion_transformer_forward_amd as W
    from video_diffusion_transformer_forward_amd import _native as N

    if args.vae_only:
        print(json.dumps({"vae_decode": time_vae()}), flush=True)
        return
    cfg = S.get_config(args.config)
    assert cfg.mode == "bf16"
    print(f"[bench] building inputs for {cfg.name}", file=sys.stderr, flush=True)
    mw = S.model_weights(cfg)
    blocks = [W.DeviceBlock(cfg, S.block_weights(cfg, b)) for b in range(cfg.n_blocks)]
    model = W.DeviceModel(cfg, mw, blocks)
    z0 = torch.from_numpy(S.latent(cfg)).cuda()
    cond = S.condition(cfg)
    cond = torch.from_numpy(cond).cuda() if cond is not None else None
    et = W.elem_dtype(cfg)
    ctx_c = torch.from_numpy(S.context(cfg, "cond")).to(et).cuda()
    ctx_n = torch.from_numpy(S.context(cfg, "null")).to(et).cuda()
    ws = W.workspace(cfg, N.ENTRY_STEP)
    z = z0.clone()
    torch.cuda.synchronize()

    def step():
        W.denoise_step(cfg, model, z, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale, ws)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    W.timing_enable(True)
    for k in range(4):
        W.timing_read(k, reset=True)
    print("[bench] timed steps", file=sys.stderr, flush=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with ClockSampler() as clocks:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(args.steps):
            step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    W.timing_enable(False)
    kt = {k: W.timing_read(c) for k, c in (("self_attention", N.KERNEL_SELF_ATTENTION),
                                           ("cross_attention", N.KERNEL_CROSS_ATTENTION),
                                           ("gemm", N.KERNEL_GEMM), ("elementwise", N.KERNEL_ELEMENTWISE))}
    assert bool(torch.isfinite(z).all())

    # the same step captured once into a HIP graph (torch.cuda.CUDAGraph on the library's
    # launches) and replayed: the kernels are the same, the host launches and the gaps between
    # them go; one replay from z0 is checked bit for bit against one eager step from z0
    graph = None
    if not args.no_graph:
        print("[bench] graph replay", file=sys.stderr, flush=True)
        zg = z0.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            W.denoise_step(cfg, model, zg, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale, ws)
        zg.copy_(z0)
        g.replay()
        ze = z0.clone()
        W.denoise_step(cfg, model, ze, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale, ws)
        torch.cuda.synchronize()
        same = bool(torch.equal(zg, ze))
        del ze
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph = {"ms_per_step": round((time.perf_counter() - tg) / args.steps * 1e3, 3),
                 "bitwise_equal_to_eager": same}
        assert bool(torch.isfinite(zg).all())
        del g, zg
        torch.cuda.empty_cache()
    # the same step in the 8-bit forms (same weights): 8-bit self-attention scores
    # (WAN_BF16_QK8), and 8-bit projections on top (WAN_FP8)
    def time_variant(cfg8, reps=3):
        ws8 = W.workspace(cfg8, N.ENTRY_STEP)
        z8 = z0.clone()
        W.denoise_step(cfg8, model, z8, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale, ws8)
        torch.cuda.synchronize()
        W.timing_enable(True)
        for k in range(4):
            W.timing_read(k, reset=True)
        t1 = time.perf_counter()
        for _ in range(reps):
            W.denoise_step(cfg8, model, z8, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale, ws8)
        torch.cuda.synchronize()
        ms8 = (time.perf_counter() - t1) / reps * 1e3
        W.timing_enable(False)
        kt8 = {k: W.timing_read(c) for k, c in (("self_attention", N.KERNEL_SELF_ATTENTION),
                                                ("cross_attention", N.KERNEL_CROSS_ATTENTION),
                                                ("gemm", N.KERNEL_GEMM), ("elementwise", N.KERNEL_ELEMENTWISE))}
        assert bool(torch.isfinite(z8).all())
        a8_ms, a8_n = kt8["self_attention"]
        del z8, ws8
        torch.cuda.empty_cache()
        return {"ms_per_step": round(ms8, 3),
                "kernel_ms_per_step": {k: round(v[0] / reps, 3) for k, v in kt8.items()},
                "self_attention_avg_launch_ms": round(a8_ms / max(a8_n, 1), 4)}

    qk8 = fp8 = None
    if not args.no_qk8:
        print("[bench] 8-bit variants", file=sys.stderr, flush=True)
        qk8 = time_variant(cfg.with_(qk8=True))
        fp8 = time_variant(cfg.with_(fp8=True))
    # diffusion cache: one step in each mode (after a store step), timed alone
    cache_ms = None
    if not args.no_cache_modes:
        cache = W.diffusion_cache(cfg, cfg.n_blocks)
        modes = {"store": N.CACHE_STORE, "reuse_attn": N.CACHE_REUSE_ATTN, "reuse_uncond": N.CACHE_REUSE_UNCOND,
                 "reuse_attn_uncond": N.CACHE_REUSE_ATTN | N.CACHE_REUSE_UNCOND}
        zc = z0.clone()
        W.denoise_step_cached(cfg, model, zc, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale,
                              N.CACHE_STORE, cache, ws)
        cache_ms = {}
        for name, mode in modes.items():
            W.denoise_step_cached(cfg, model, zc, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale,
                                  mode, cache, ws)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(2):
                W.denoise_step_cached(cfg, model, zc, cond, ctx_c, ctx_n, cfg.timestep, cfg.dt, cfg.guide_scale,
                                      mode, cache, ws)
            torch.cuda.synchronize()
            cache_ms[name] = round((time.perf_counter() - t1) / 2 * 1e3, 3)
        cache_gb = round(cache.numel() / 1e9, 3)
        del cache
        torch.cuda.empty_cache()
    if args.calib_copy:
        src = torch.ones(CALIB_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms_step = elapsed / args.steps * 1e3
    flops = step_flops(cfg)
    tflops = flops / (ms_step * 1e-3) / 1e12
    bf = block_flops(cfg, 2 * cfg.batch)
    attn_ms, attn_n = kt["self_attention"]
    attn_avg = attn_ms / max(attn_n, 1)
    attn_achieved = bf["self_attention"] / (attn_avg * 1e-3) / 1e12
    per_block_ms = ms_step / cfg.n_blocks
    block_tflops = sum(bf.values()) / (per_block_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "step_ms_events": {"median": round(step_ms[len(step_ms) // 2], 3), "min": round(step_ms[0], 3),
                           "max": round(step_ms[-1], 3)},
        "clocks_during_timed_steps": clocks.summary(),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents/context, N(0,0.02) random-init weights)",
        "config": {"workload": f"{cfg.name}: one CFG denoise step of the 1.3B DiT, latent 16x{cfg.frames}x"
                               f"{cfg.height}x{cfg.width} (480p x 81 frames), L={cfg.seq_len}, D={cfg.dim}, "
                               f"{cfg.heads}x{cfg.head_dim} heads, FFN {cfg.ffn_dim}, {cfg.n_blocks} blocks, "
                               f"CFG batch 2, {cfg.txt_len} text tokens",
                   "global_batch": 2 * cfg.batch, "seq_len": cfg.seq_len, "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * tflops / MI355X_BF16_TFLOPS, 2),
        "ms_per_block_forward_cfg_batch": round(per_block_ms, 3),
        "block_tflops": round(block_tflops, 2),
        "step_tflop": round(flops / 1e12, 3),
        "kernel_ms_per_step": {k: round(v[0] / args.steps, 3) for k, v in kt.items()},
        "roofline": {"bound": "mfma", "kernel": "self-attention (attn_self_wide_kernel<128,3,1,8,true>, static offset, and its flagged-workgroup pass)",
                     "achieved": round(attn_achieved, 2), "peak": MI355X_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_achieved / MI355X_BF16_TFLOPS, 4), "traffic": attn_traffic_bytes(),
                     "traffic_unit": "bytes per launch (L2-memory fetch + write counters)",
                     "algorithmic_bytes": 4 * 2 * cfg.batch * cfg.heads * cfg.seq_len * cfg.head_dim * 2,
                     "avg_launch_ms": round(attn_avg, 4), "launches": attn_n,
                     "flop_per_launch": bf["self_attention"]},
    }
    for key, var, note in (
            ("qk8_step", qk8, "self-attention scores from e4m3 q and k (per-token power-of-two scales); P V, "
                              "GEMMs and the rest stay bf16"),
            ("fp8_step", fp8, "as qk8_step, plus e4m3 q/k/v, cross-attention query and FFN projections "
                              "(power-of-two scales per 128-block of both operands, weights quantised inside the "
                              "step); output projections, context K/V and attention P V stay bf16")):
        if var is None:
            continue
        a8 = var["self_attention_avg_launch_ms"]
        var.update({
            "tflops_equivalent": round(flops / (var["ms_per_step"] * 1e-3) / 1e12, 2),
            "speedup_vs_bf16_step": round(ms_step / var["ms_per_step"], 4),
            "self_attention_speedup": round(attn_avg / a8, 4) if a8 > 0 else None,
            "note": note + "; reduced-precision variant, not the headline value"})
        out[key] = var
    if graph is not None:
        graph.update({"tflops": round(flops / (graph["ms_per_step"] * 1e-3) / 1e12, 2),
                      "note": "the timed step captured once into a HIP graph and replayed (same kernels, no "
                              "host launches); not the headline value"})
        out["graph_step"] = graph
    if cache_ms is not None:
        out["diffusion_cache"] = {
            "ms_per_step": cache_ms, "cache_gb": cache_gb,
            "note": "one CFG step per mode after a store step; a reuse step skips the QKV projection and "
                    "self-attention (reuse_attn) and/or the unconditional branch (reuse_uncond)"}
    if not args.no_vae:
        print("[bench] vae decode", file=sys.stderr, flush=True)
        out["vae_decode"] = time_vae()
        print("[bench] streaming queue", file=sys.stderr, flush=True)
        out["stream"] = time_stream(cfg, model, ctx_c)
    if args.block_configs:
        out["blocks"] = {}
        for name in [c for c in args.block_configs.split(",") if c]:
            print(f"[bench] block {name}", file=sys.stderr, flush=True)
            out["blocks"][name] = time_block(S.get_config(name))
    if args.vendor_gemms:
        print("[bench] vendor GEMMs", file=sys.stderr, flush=True)
        out["vendor_gemms"] = time_vendor_gemms(cfg)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
