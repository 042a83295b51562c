"""Seeded synthetic inputs for the SPD draft-and-verify cycle.

This module is shared by the tests, the bench and the oracle checks.  It holds
none of the method's arithmetic: it only draws seeded random tensors of the
shapes the pages use (pseudo-random normals/uniforms from torch generators,
raw 64-bit words from numpy's Philox4x64-10) and rounds them to the storage
dtype with torch's round-to-nearest-even cast.  Probability rows for the batched
verify stress test are made with the library softmax, and drafts with the
library multinomial sampler.

Workload shapes follow "Speculative Pipeline Decoding" (arXiv 2605.30852),
section 3.2 (anchors [0,8,16,24,31] for a 32-layer target) and section 4
(Qwen3.5-4B/-9B-shaped targets, batch 1, context up to 2048, pipeline widths
4/8/16); the 50/50 saturated/partial-fill mix follows the review blog's
"simulated pipeline occupancy" paragraph.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field, replace

import numpy as np
import torch

F32 = 0
BF16 = 1
ZERO_MASK = 0
CLAMP_MIN = 1


@dataclass(frozen=True)
class SpdShape:
    """Sizes of one SPD workload."""
    name: str
    L: int                  # target layers
    n: int                  # pipeline stages
    anchors: tuple          # anchor layers B
    d: int                  # hidden size (target and PDM)
    Ls: int                 # PDM decoder layers
    Hq: int
    Hkv: int
    hd: int
    dff: int
    V: int
    dtype: int              # F32 or BF16 storage of weights/anchors/KV
    ctx: int                # context length t at the measured cycle
    temperature: float
    lm_std: float           # std of both LM heads' weights
    mix: bool = False       # 50% saturated / 50% partial-fill cycles
    anchor_mode: int = ZERO_MASK
    norm_k0: int = 0
    feature_schedule: int = 0  # 0 pre-step, 1 post-step, 2 first-stage only
    top_k: int = 0             # sampling filters at T > 0 (0 / 1.0: off)
    top_p: float = 1.0
    eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def m(self) -> int:
        return len(self.anchors)

    def with_(self, **kw) -> "SpdShape":
        return replace(self, **kw)


def _shapes():
    a32 = (0, 8, 16, 24, 31)
    tiny = SpdShape("tiny_fp32_n4", L=8, n=4, anchors=(0, 4, 7), d=64, Ls=1, Hq=4, Hkv=4,
                    hd=16, dff=256, V=512, dtype=F32, ctx=32, temperature=0.0, lm_std=0.02)
    b4_n4 = SpdShape("qwen35_4b_n4_ls1_greedy", L=32, n=4, anchors=a32, d=2560, Ls=1, Hq=20,
                     Hkv=4, hd=128, dff=9728, V=151936, dtype=BF16, ctx=2048,
                     temperature=0.0, lm_std=0.02)
    b4_n8 = SpdShape("qwen35_4b_n8_ls2_t1_mix", L=32, n=8, anchors=a32, d=2560, Ls=2, Hq=20,
                     Hkv=4, hd=128, dff=9728, V=151936, dtype=BF16, ctx=2048,
                     temperature=1.0, lm_std=3.0 / np.sqrt(2560), mix=True)
    b9_n16 = SpdShape("qwen35_9b_n16_ls4_t1", L=32, n=16, anchors=a32, d=4096, Ls=4, Hq=32,
                      Hkv=8, hd=128, dff=12288, V=151936, dtype=BF16, ctx=4096,
                      temperature=1.0, lm_std=3.0 / np.sqrt(4096))
    return {s.name: s for s in (tiny, b4_n4, b4_n8, b9_n16)}


SHAPES = _shapes()
TINY = SHAPES["tiny_fp32_n4"]
HEADLINE = SHAPES["qwen35_4b_n8_ls2_t1_mix"]


@dataclass(frozen=True)
class VerifyShape:
    name: str = "verify_b64_g7"
    B: int = 64
    gamma: int = 7
    V: int = 151936
    logit_std: float = 3.0
    noise_std: float = 1.0
    bonus: int = 1
    temperature: float = 1.0


VERIFY_STRESS = VerifyShape()


# ---------------------------------------------------------------- generators

def _seed(base: int, name: str) -> int:
    return (int(base) * 1_000_003 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF


def _gen(device, base: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(base, name))
    return g


def storage_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def normal(shape, std, *, device, seed, name, dtype=torch.float32):
    g = _gen(device, seed, name)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform(shape, lo, hi, *, device, seed, name, dtype=torch.float32):
    g = _gen(device, seed, name)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(hi - lo).add_(lo)
    return x.to(dtype)


def rand_words(seed: int, stream: int, count: int) -> np.ndarray:
    """`count` raw 64-bit words of numpy's Philox4x64-10 keyed by (seed, stream)."""
    bitgen = np.random.Philox(key=(int(seed) << 32) | int(stream))
    return bitgen.random_raw(count).astype(np.uint64)


@dataclass
class CycleInputs:
    """Device-resident weights and synthetic target states for one shape."""
    shape: SpdShape
    store_layers: list
    store: torch.Tensor          # [T_cap][S][d] anchor hidden states H_i^l
    h_final: torch.Tensor        # [T_cap][d]   float32 target last-layer states (already final-normed)
    fc_norm: torch.Tensor        # [m*d]
    w_fc: torch.Tensor           # [d][m*d]
    layers: list = field(default_factory=list)  # dicts of per-layer tensors
    final_norm: torch.Tensor = None
    w_dlm: torch.Tensor = None   # [V][d] draft LM head
    w_tlm: torch.Tensor = None   # [V][d] target LM head
    T_cap: int = 0


def layer_weights(s: SpdShape, li: int, *, device, seed):
    dt = storage_dtype(s.dtype)
    kw = dict(device=device, seed=seed, dtype=dt)
    nq = (s.Hq + 2 * s.Hkv) * s.hd
    return {
        "attn_norm": uniform((s.d,), 0.5, 1.5, name=f"l{li}.attn_norm", **kw),
        "wqkv": normal((nq, s.d), 0.02, name=f"l{li}.wqkv", **kw),
        "q_norm": uniform((s.hd,), 0.5, 1.5, name=f"l{li}.q_norm", **kw),
        "k_norm": uniform((s.hd,), 0.5, 1.5, name=f"l{li}.k_norm", **kw),
        "wo": normal((s.d, s.Hq * s.hd), 0.02, name=f"l{li}.wo", **kw),
        "mlp_norm": uniform((s.d,), 0.5, 1.5, name=f"l{li}.mlp_norm", **kw),
        "w_gate_up": normal((2 * s.dff, s.d), 0.02, name=f"l{li}.w_gate_up", **kw),
        "w_down": normal((s.d, s.dff), 0.02, name=f"l{li}.w_down", **kw),
    }


def cycle_inputs(s: SpdShape, store_layers, *, device, seed=0, T_cap=None, with_heads=True) -> CycleInputs:
    """Seeded weights and target states of shape `s`.  `store_layers` lists the
    target layers the anchor store holds, in slot order; it is the caller's (the
    oracle's or the library's slot table), so that this module does none of the
    method's arithmetic."""
    dt = storage_dtype(s.dtype)
    T_cap = int(T_cap or (s.ctx + 64))
    sl = [int(x) for x in store_layers]
    store = normal((T_cap, len(sl), s.d), 1.0, device=device, seed=seed + 1, name="anchors", dtype=dt)
    h_final = normal((T_cap, s.d), 1.0, device=device, seed=seed + 1, name="h_final")
    ci = CycleInputs(
        shape=s, store_layers=sl, store=store, h_final=h_final,
        fc_norm=uniform((s.m * s.d,), 0.5, 1.5, device=device, seed=seed, name="fc_norm", dtype=dt),
        w_fc=normal((s.d, s.m * s.d), 0.02, device=device, seed=seed, name="w_fc", dtype=dt),
        layers=[layer_weights(s, li, device=device, seed=seed) for li in range(s.Ls)],
        final_norm=uniform((s.d,), 0.5, 1.5, device=device, seed=seed, name="final_norm", dtype=dt),
        T_cap=T_cap,
    )
    if with_heads:
        ci.w_dlm = normal((s.V, s.d), s.lm_std, device=device, seed=seed, name="w_dlm", dtype=dt)
        ci.w_tlm = normal((s.V, s.d), s.lm_std, device=device, seed=seed, name="w_tlm", dtype=dt)
    return ci


def cycle_schedule(s: SpdShape, n_cycles: int, seed: int = 2):
    """In-flight count a for each independent cycle.  Without the mix every cycle
    is saturated (a = n).  With it, word 3 of each Philox block decides: top bit
    0 -> saturated, else a = 1 + ((w >> 32) mod (n-1))."""
    if not s.mix:
        return [s.n] * n_cycles
    w = rand_words(seed, 2, 4 * n_cycles).reshape(n_cycles, 4)[:, 3]
    out = []
    for x in w.tolist():
        if (x >> 63) == 0:
            out.append(s.n)
        else:
            out.append(1 + ((x >> 32) % (s.n - 1)))
    return out


def draft_row_logits(V, std, *, device, seed, name):
    """Stand-in draft logits for the token under verification when cycles are
    run independently (the ring row a trajectory would hold)."""
    return normal((V,), std, device=device, seed=seed, name=name)


def verify_stress_inputs(v: VerifyShape, *, device, seed=3):
    """Batched verify stress: p_logits ~ N(0, std^2); q_logits = p_logits + N(0, noise^2)
    per row; fp32 library softmax; drafts x_j ~ q_j by the library sampler;
    64-bit words [B][gamma+1][2]."""
    B, G, V = v.B, v.gamma, v.V
    pl = normal((B, G + v.bonus, V), v.logit_std, device=device, seed=seed, name="p_logits")
    noise = normal((B, G, V), v.noise_std, device=device, seed=seed, name="q_noise")
    ql = pl[:, :G, :] + noise
    del noise
    p = torch.softmax(pl / v.temperature, dim=-1).float().contiguous()
    q = torch.softmax(ql / v.temperature, dim=-1).float().contiguous()
    del pl, ql
    g = _gen(device, seed, "drafts")
    draft = torch.multinomial(q.reshape(B * G, V), 1, generator=g).reshape(B, G).to(torch.int32)
    words = rand_words(seed, 1, B * (G + 1) * 2).reshape(B, G + 1, 2)
    return p, q, draft.contiguous(), words


def kv_cache(s: SpdShape, T_cap: int, *, device, seed=4):
    """Committed key/value cache contents for a cycle run without prefill:
    keys [Ls][Hkv][T_cap][hd] (position-major) and values [Ls][Hkv][hd][T_cap]
    (position-minor), N(0,1) in the storage dtype."""
    dt = storage_dtype(s.dtype)
    k = normal((s.Ls, s.Hkv, T_cap, s.hd), 1.0, device=device, seed=seed, name="k_cache", dtype=dt)
    v = normal((s.Ls, s.Hkv, s.hd, T_cap), 1.0, device=device, seed=seed, name="v_cache", dtype=dt)
    return k, v


def cycle_words(n_cycles: int, seed: int = 2, stream: int = 0) -> np.ndarray:
    """One 4-word block per cycle: word 0 -> accept uniform, word 1 -> resample
    uniform, word 2 -> draft-sampling uniform, word 3 -> harness draws."""
    return rand_words(seed, stream, 4 * n_cycles).reshape(n_cycles, 4)


def words_tensor(words: np.ndarray, device) -> torch.Tensor:
    """uint64 words as an int64 tensor with the same bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int64)).to(device)
