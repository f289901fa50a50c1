"""Seeded synthetic inputs for the routed-expert FP8 grouped-matmul workloads.

Shared by the tests, the benchmark and the smoke check; used to feed both the
HIP library and the CPU oracle.  It holds none of the method's arithmetic: it
draws random numbers, rounds them to bf16 and prepares e4m3fn weight codes with
torch's own float8 cast (a library routine), because the method receives its
weights already quantized (the weight codes and a per-output-channel f32 scale
are inputs of every call).

Every array comes from ``numpy.random.Generator(PCG64(SeedSequence([config,
stream])))`` so each tensor of each workload is reproducible on its own.

Workloads (sizes from the task's five configurations):

====  =====================================================================
0     tiny forward: G=4, M=256, K=128, N=256; sizes = random composition
1     wi forward + SwiGLU: G=8, M=8192 (1024 tokens x top-8 uniform
      routing), K=2048, N=2x768; activations N(0,1) with 1% outliers x50
2     wo forward and dLHS: G=8, M=8192, K=768, N=2048; dout N(0, 1e-3)
3     dropless per-device shape: G=32, static M=32768 with 19,661 valid
      rows, Zipf(1.1)-skewed sizes with four empty experts; wi K=7168,
      N=2x2048; wo K=2048, N=7168; stale tail rows hold Inf/NaN garbage
4     tgmm on the config-3 buffer: lhs [32768, 7168], dout [32768, 2048],
      tile_m = 512
====  =====================================================================

The fused dSwiGLU backward and the FFN forward/backward reuse these shapes
(``dswiglu`` and ``ffn`` below): the wi pre-activation [gate | up] is drawn
N(0, 2^2) in bf16, so every region of silu' (its zero near -1.28, the
saturated tails) is populated.
"""
from __future__ import annotations

import numpy as np
import torch

#: stale-row garbage cycled through the rows past the valid prefix:
#: +Inf, -Inf, NaN, NaN (all ones), largest finite bf16
GARBAGE_BF16 = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFFF, 0x7F7F], dtype=np.uint16)

# stream ids, one per tensor role
ROUTING, LHS_WI, LHS_WO, OUTLIERS_WI, OUTLIERS_WO, W_WI, W_WO, DOUT_WI, DOUT_WO, LHS, DOUT = range(11)
PREACT, FFN_X, FFN_X_OUT, FFN_WI, FFN_WO, FFN_DY = range(11, 17)

SHAPES = {
    0: dict(G=4, M=256, K=128, N=256),
    1: dict(G=8, M=8192, K=2048, N=1536),
    2: dict(G=8, M=8192, K=768, N=2048),
    3: dict(G=32, M=32768, valid=19661, K_wi=7168, N_wi=4096, K_wo=2048, N_wo=7168),
    4: dict(G=32, M=32768, valid=19661, K=7168, N=2048, tile_m=512),
}


def rng(config: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(config), int(stream)])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 values (torch's round-to-nearest-even cast)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    step = 1 << 26
    for i in range(0, flat_in.size, step):
        t = torch.from_numpy(flat_in[i:i + step]).to(torch.bfloat16)
        flat_out[i:i + step] = t.view(torch.int16).numpy().view(np.uint16)
    return out


def weight_codes(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """e4m3fn codes and per-output-channel f32 scales of one expert's weight
    ``w[K, N]``: scale = absmax over K / 448, codes = torch's e4m3fn cast of
    ``w / scale`` (clamped to +-448 first, since that cast does not saturate)."""
    w = np.asarray(w, dtype=np.float32)
    absmax = np.max(np.abs(w), axis=0)
    scale = (absmax / np.float32(448.0)).astype(np.float32)
    q = np.clip(w / scale[None, :], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def weights(config: int, stream: int, G: int, K: int, N: int, std: float = 0.02):
    """Weights ~ N(0, std) per expert, as (codes [G,K,N] uint8, scale [G,N] f32)."""
    r = rng(config, stream)
    codes = np.empty((G, K, N), dtype=np.uint8)
    scale = np.empty((G, N), dtype=np.float32)
    for g in range(G):
        w = r.standard_normal((K, N), dtype=np.float32) * np.float32(std)
        codes[g], scale[g] = weight_codes(w)
    return codes, scale


def group_sizes(config: int, variant: str | None = None) -> np.ndarray:
    """Expert row counts of a workload (int32 [G])."""
    r = rng(config, ROUTING)
    if config == 0:
        if variant == "forced":
            return np.array([0, 100, 156, 0], dtype=np.int32)
        cuts = np.sort(r.integers(0, 257, size=3))
        return np.diff(np.concatenate([[0], cuts, [256]])).astype(np.int32)
    if config in (1, 2):
        if variant == "balanced":
            return np.full(8, 1024, dtype=np.int32)
        slots = r.integers(0, 8, size=1024 * 8)          # each token-slot's expert
        return np.bincount(slots, minlength=8).astype(np.int32)
    if config in (3, 4):
        G, valid = 32, SHAPES[3]["valid"]
        r3 = rng(3, ROUTING)                              # configs 3 and 4 share the buffer
        interior = r3.choice(np.arange(1, 31), size=2, replace=False)
        empty = np.concatenate([[0, 31], interior])
        live = np.setdiff1d(np.arange(G), empty)
        ranks = r3.permutation(len(live)) + 1
        p = 1.0 / ranks.astype(np.float64) ** 1.1
        p /= p.sum()
        sizes = np.zeros(G, dtype=np.int64)
        sizes[live] = r3.multinomial(valid, p)
        return sizes.astype(np.int32)
    raise ValueError(config)


def activations(config: int, stream: int, M: int, K: int, valid: int,
                outlier_stream: int | None = None) -> np.ndarray:
    """bf16 [M, K]: rows < valid ~ N(0,1) (optionally 1% of entries x50, chosen
    without replacement); rows >= valid hold the garbage cycle."""
    r = rng(config, stream)
    x = r.standard_normal((valid, K), dtype=np.float32)
    if outlier_stream is not None and valid * K > 0:
        ro = rng(config, outlier_stream)
        idx = ro.choice(valid * K, size=(valid * K) // 100, replace=False)
        x.reshape(-1)[idx] *= np.float32(50.0)
    out = np.empty((M, K), dtype=np.uint16)
    out[:valid] = to_bf16_bits(x)
    fill_garbage(out, valid)
    return out


def gradients(config: int, stream: int, M: int, N: int, valid: int, std: float = 1e-3) -> np.ndarray:
    """bf16 [M, N] output gradients ~ N(0, std) on valid rows, garbage after."""
    r = rng(config, stream)
    d = r.standard_normal((valid, N), dtype=np.float32) * np.float32(std)
    out = np.empty((M, N), dtype=np.uint16)
    out[:valid] = to_bf16_bits(d)
    fill_garbage(out, valid)
    return out


def fill_garbage(buf: np.ndarray, valid: int) -> None:
    """Overwrite rows >= valid with the Inf/NaN/max garbage cycle."""
    tail = buf[valid:].reshape(-1)
    if tail.size:
        tail[:] = np.resize(GARBAGE_BF16, tail.size)


def make(config: int, op: str, variant: str | None = None) -> dict:
    """Inputs of one op of one workload.

    ops: ``fwd`` (config 0), ``wi`` (configs 1, 3: SwiGLU forward), ``wo``
    (configs 2, 3), ``dlhs_wo`` (configs 2, 3), ``dlhs_wi`` (config 3),
    ``dequant`` (any config with wo or plain weights), ``tgmm`` (config 4).
    """
    gs = group_sizes(config, variant)
    sh = SHAPES[config]
    if config == 0:
        G, M, K, N = sh["G"], sh["M"], sh["K"], sh["N"]
        codes, scale = weights(0, W_WO, G, K, N)
        d = dict(G=G, M=M, K=K, N=N, group_sizes=gs, codes=codes, scale=scale)
        if op in ("fwd", "wo"):
            d["lhs"] = activations(0, LHS, M, K, M)
        elif op in ("dlhs", "dlhs_wo"):
            d["dout"] = gradients(0, DOUT, M, N, M)
        elif op != "dequant":
            raise ValueError(op)
        return d
    if config in (1, 2):
        G, M, K, N = sh["G"], sh["M"], sh["K"], sh["N"]
        wstream = W_WI if config == 1 else W_WO
        codes, scale = weights(config, wstream, G, K, N)
        d = dict(G=G, M=M, K=K, N=N, group_sizes=gs, codes=codes, scale=scale)
        if op in ("wi", "wo", "fwd"):
            d["lhs"] = activations(config, LHS, M, K, M, outlier_stream=OUTLIERS_WI)
        elif op in ("dlhs_wo", "dlhs"):
            d["dout"] = gradients(config, DOUT, M, N, M)
        elif op != "dequant":
            raise ValueError(op)
        return d
    if config == 3:
        G, M, valid = sh["G"], sh["M"], sh["valid"]
        if op in ("wi", "dlhs_wi"):
            K, N, wstream = sh["K_wi"], sh["N_wi"], W_WI
        elif op in ("wo", "dlhs_wo", "dequant"):
            K, N, wstream = sh["K_wo"], sh["N_wo"], W_WO
        else:
            raise ValueError(op)
        codes, scale = weights(3, wstream, G, K, N)
        d = dict(G=G, M=M, K=K, N=N, valid=valid, group_sizes=gs, codes=codes, scale=scale)
        if op == "wi":
            d["lhs"] = activations(3, LHS_WI, M, K, valid, outlier_stream=OUTLIERS_WI)
        elif op == "wo":
            d["lhs"] = activations(3, LHS_WO, M, K, valid, outlier_stream=OUTLIERS_WO)
        elif op == "dlhs_wi":
            d["dout"] = gradients(3, DOUT_WI, M, N, valid)
        elif op == "dlhs_wo":
            d["dout"] = gradients(3, DOUT_WO, M, N, valid)
        return d
    if config == 4:
        if op != "tgmm":
            raise ValueError(op)
        G, M, valid, K, N = sh["G"], sh["M"], sh["valid"], sh["K"], sh["N"]
        return dict(G=G, M=M, K=K, N=N, valid=valid, tile_m=sh["tile_m"], group_sizes=gs,
                    lhs=activations(4, LHS, M, K, valid, outlier_stream=OUTLIERS_WI),
                    dout=gradients(4, DOUT, M, N, valid))
    raise ValueError(config)


def preactivations(config: int, M: int, I2: int, valid: int, std: float = 2.0) -> np.ndarray:
    """bf16 [M, 2I] wi pre-activations ~ N(0, std) on valid rows, garbage after."""
    r = rng(config, PREACT)
    z = r.standard_normal((valid, I2), dtype=np.float32) * np.float32(std)
    out = np.empty((M, I2), dtype=np.uint16)
    out[:valid] = to_bf16_bits(z)
    fill_garbage(out, valid)
    return out


#: FFN / dSwiGLU shapes: small (ragged, static tail), config 2's wo, config 3's
FFN_SHAPES = {
    "small": dict(G=4, M=320, valid=None, H=256, I=256),
    "small128": dict(G=4, M=320, valid=None, H=256, I=128),
    "small384": dict(G=4, M=320, valid=None, H=384, I=128),
    2: dict(G=8, M=8192, valid=8192, H=2048, I=768),
    3: dict(G=32, M=32768, valid=SHAPES[3]["valid"], H=7168, I=2048),
}


def _ffn_sizes(key):
    sh = FFN_SHAPES[key]
    if key in ("small", "small128", "small384"):
        r = rng(90, ROUTING)
        cuts = np.sort(r.integers(0, 257, size=2))
        parts = np.diff(np.concatenate([[0], cuts, [256]]))
        return np.array([parts[0], 0, parts[1], parts[2]], dtype=np.int32)   # one empty expert
    return group_sizes(key)


def dswiglu(key) -> dict:
    """Inputs of the fused wo dLHS + dSwiGLU: dout [M, H] ~ N(0, 1e-3), wo codes
    [G, I, H], preact [M, 2I] ~ N(0, 4); stale rows hold garbage."""
    sh = FFN_SHAPES[key]
    G, M, H, I = sh["G"], sh["M"], sh["H"], sh["I"]
    gs = _ffn_sizes(key)
    valid = int(gs.sum())
    c = 90 if key in ("small", "small128") else key
    codes, scale = weights(c, W_WO, G, I, H)
    return dict(G=G, M=M, K=I, N=H, valid=valid, group_sizes=gs, codes=codes, scale=scale,
                dout=gradients(c, DOUT_WO, M, H, valid), preact=preactivations(c, M, 2 * I, valid))


def ffn(key) -> dict:
    """Inputs of one routed-expert FFN forward + backward: x [M, H] ~ N(0, 1)
    with 1% outliers x50, wi [G, H, 2I] and wo [G, I, H] ~ N(0, 0.02) as
    codes + scales, dy [M, H] ~ N(0, 1e-3); stale rows hold garbage."""
    sh = FFN_SHAPES[key]
    G, M, H, I = sh["G"], sh["M"], sh["H"], sh["I"]
    gs = _ffn_sizes(key)
    valid = int(gs.sum())
    c = 91 if key in ("small", "small128", "small384") else key
    wi_codes, wi_scale = weights(c, FFN_WI, G, H, 2 * I)
    wo_codes, wo_scale = weights(c, FFN_WO, G, I, H)
    return dict(G=G, M=M, H=H, I=I, valid=valid, group_sizes=gs, wi_codes=wi_codes, wi_scale=wi_scale,
                wo_codes=wo_codes, wo_scale=wo_scale,
                x=activations(c, FFN_X, M, H, valid, outlier_stream=FFN_X_OUT),
                dy=gradients(c, FFN_DY, M, H, valid))


def bf16_weights(config: int, stream: int, G: int, K: int, N: int, std: float = 0.02) -> np.ndarray:
    """bf16 weights [G, K, N] ~ N(0, std) for the bf16 measurement arm."""
    r = rng(config, stream)
    out = np.empty((G, K, N), dtype=np.uint16)
    for g in range(G):
        out[g] = to_bf16_bits(r.standard_normal((K, N), dtype=np.float32) * np.float32(std))
    return out


#: The pages' GMM kernel microbenchmark at the trainer's per-device shapes: one
#: call at full fill, 64 experts, 225,280 rows; wi 4096 -> 2x1024, wo 1024 -> 4096.
MICRO = dict(G=64, M=225280, H=4096, I=1024)
MICRO_CONFIG = 7
MICRO_CHUNK = 8192


def micro_group_sizes() -> np.ndarray:
    """Full fill: every row valid; each row's expert uniform over the 64."""
    r = rng(MICRO_CONFIG, ROUTING)
    return np.bincount(r.integers(0, MICRO["G"], size=MICRO["M"]), minlength=MICRO["G"]).astype(np.int32)


def _torch_gen(*key) -> torch.Generator:
    """CPU torch generator seeded from a SeedSequence of ``key`` (the large
    microbenchmark tensors use torch's CPU normal sampler, several times
    faster than numpy's here; reproducible for a given torch version)."""
    seed = int(np.random.SeedSequence(list(key)).generate_state(1, dtype=np.uint64)[0] >> 1)
    return torch.Generator().manual_seed(seed)


def micro_rows(stream: int, K: int, outliers: bool = True) -> np.ndarray:
    """bf16 [225280, K]: activations N(0,1) with 1% of the entries (positions
    drawn with replacement) x50, or with outliers=False gradients N(0, 1e-3)."""
    M = MICRO["M"]
    g = _torch_gen(MICRO_CONFIG, stream)
    x = torch.randn((M, K), generator=g)
    if outliers:
        flat = x.view(-1)
        idx = torch.randint(0, flat.numel(), (flat.numel() // 100,), generator=g)
        flat[idx] = flat[idx] * 50.0
    else:
        x *= 1e-3
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def micro_weights(stream: int, G: int, K: int, N: int, std: float = 0.02):
    """Weights ~ N(0, std) per expert as e4m3 codes + per-channel scales
    (the recipe of ``weight_codes``), drawn with a torch CPU generator."""
    g = _torch_gen(MICRO_CONFIG, stream)
    codes = np.empty((G, K, N), dtype=np.uint8)
    scale = np.empty((G, N), dtype=np.float32)
    for e in range(G):
        w = torch.randn((K, N), generator=g) * std
        s = w.abs().amax(dim=0) / 448.0                    # f32, as weight_codes
        q = (w / s[None, :]).clamp(-448.0, 448.0)
        codes[e] = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scale[e] = s.numpy()
    return codes, scale


def micro(op: str) -> dict:
    """Inputs of one microbenchmark GMM: op ``wi`` (K=4096, N=2x1024, SwiGLU) or
    ``wo`` (K=1024, N=4096), with e4m3 codes + scales as in config 0."""
    G, H, I = MICRO["G"], MICRO["H"], MICRO["I"]
    K, N, ws, xs = (H, 2 * I, W_WI, LHS_WI) if op == "wi" else (I, H, W_WO, LHS_WO)
    codes, scale = micro_weights(ws, G, K, N)
    return dict(G=G, M=MICRO["M"], K=K, N=N, group_sizes=micro_group_sizes(), codes=codes, scale=scale,
                lhs=micro_rows(xs, K))
