"""Seeded synthetic inputs for the MoE token permute / unpermute path.

This module is shared by the tests, the smoke check and the benchmark.  It
holds no part of the permute / unpermute arithmetic: it only draws routing
decisions (expert ids and their weights), activations and expert outputs with
the shapes and distributions of the workloads, and quantises activations to
fp8 codes where a workload asks for fp8 input.

Recipe (every workload, seed 0 unless a test says otherwise):

* One ``numpy.random.SeedSequence(seed)`` is split with ``spawn`` into
  independent streams: routing, routing weights, activation, expert output.
* Routing is drawn on the host with numpy:
    - ``uniform``: a uniformly random ordered set of ``topk`` distinct experts
      per token (the first ``topk`` entries of a random permutation);
    - ``softmax_topk``: N(0,1) router logits ``[N, E]``, softmax in float64,
      the ``topk`` largest probabilities in descending order (ties go to the
      lower expert id), weights renormalised over the chosen ``topk``;
    - ``zipf``: expert popularity proportional to ``rank^-s`` with ranks from
      a seeded permutation, and popularity zero for a seeded set of experts
      that always holds expert 0 and expert E-1; ``topk`` distinct experts per
      token are drawn by successive sampling without replacement (draw,
      remove, renormalise), realised as exponential races: each expert gets
      the key ``Exp(1) / p_e`` and the ``topk`` smallest keys, in ascending
      order, are the draws in order.
  Weights for ``uniform`` and ``zipf`` are the softmax of N(0,1) logits over
  the chosen experts.  Weights are float32.
* Activations and expert outputs are N(0,1) float32 from a torch generator on
  the requested device, seeded from the same SeedSequence, then cast to the
  workload's type (bfloat16 by round-to-nearest-even).  The same seed gives
  different numbers on the host and on a GPU; every comparison hands one and
  the same tensor to both sides.
* fp8 activations: per-token scale ``max_h |x[t,h]| / 448`` (float32, 1 for an
  all-zero row), codes = OCP E4M3FN rounding of ``x / scale`` (clamped to
  +-448), stored as raw bytes.
* Expert maps (expert parallelism over ``ep_size`` ranks): ``contiguous``
  gives rank r the experts ``[r*E/ep, (r+1)*E/ep)`` in order, ``round_robin``
  the experts ``g`` with ``g % ep == r``; local ids count the owned experts in
  ascending global id; ``shuffled`` takes the contiguous set and numbers it
  in a seeded random order.  Every other expert maps to -1.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

FP8_E4M3_MAX = 448.0


@dataclass(frozen=True)
class MoEWorkload:
    name: str
    num_tokens: int
    hidden_size: int
    num_experts: int
    topk: int
    hidden_dtype: str  # "f32" | "bf16" | "fp8_e4m3"
    output_dtype: str  # "f32" | "bf16"  (expanded expert output and unpermute output)
    routing: str  # "uniform" | "softmax_topk" | "zipf"
    zipf_s: float = 0.0
    zipf_empty: int = 0

    @property
    def num_rows(self) -> int:
        return self.num_tokens * self.topk

    def with_tokens(self, n: int) -> "MoEWorkload":
        return replace(self, num_tokens=n)


WORKLOADS: dict[str, MoEWorkload] = {
    # N=16, H=128 fp32, E=8, topk=2 uniform distinct.
    "tiny": MoEWorkload("tiny", 16, 128, 8, 2, "f32", "f32", "uniform"),
    # Mixtral-shaped: N=4096, H=4096 bf16, E=8, top-2 of softmax router logits.
    "mixtral": MoEWorkload("mixtral", 4096, 4096, 8, 2, "bf16", "bf16", "softmax_topk"),
    # Qwen3-MoE-shaped: N=8192, H=2048 bf16, E=128, top-8 of softmax router logits.
    "qwen3": MoEWorkload("qwen3", 8192, 2048, 128, 8, "bf16", "bf16", "softmax_topk"),
    # DeepSeek-V3-shaped skewed routing: N=16384, H=7168 bf16, E=256, topk=8, Zipf(1.2), 16 empty experts.
    "dsv3": MoEWorkload("dsv3", 16384, 7168, 256, 8, "bf16", "bf16", "zipf", zipf_s=1.2, zipf_empty=16),
    # Small-batch decode: H=7168 fp8 codes + per-token scale, E=256, topk=8 uniform; N swept.
    "decode": MoEWorkload("decode", 256, 7168, 256, 8, "fp8_e4m3", "bf16", "uniform"),
}

DECODE_SWEEP = (1, 4, 16, 64, 256)


def expert_map_for(num_experts: int, ep_size: int, rank: int, layout: str = "contiguous", seed: int = 0):
    """(expert_map int32 [num_experts], num_local_experts) of one rank; see the module recipe."""
    if not 0 <= rank < ep_size:
        raise ValueError("rank outside [0, ep_size)")
    if layout == "round_robin":
        owned = [g for g in range(num_experts) if g % ep_size == rank]
    else:
        owned = [g for g in range(num_experts) if g * ep_size // num_experts == rank]
    if layout == "shuffled":
        owned = [owned[i] for i in np.random.default_rng(seed).permutation(len(owned))]
    elif layout not in ("contiguous", "round_robin"):
        raise ValueError("unknown layout %r" % layout)
    emap = np.full(num_experts, -1, dtype=np.int32)
    for local, g in enumerate(owned):
        emap[g] = local
    return emap, max(len(owned), 1)

ELEMENT_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    children = ss.spawn(4)
    return {
        "routing": np.random.default_rng(children[0]),
        "weights": np.random.default_rng(children[1]),
        "hidden_seed": int(children[2].generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF),
        "output_seed": int(children[3].generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF),
    }


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def zipf_popularity(num_experts: int, s: float, n_empty: int, rng: np.random.Generator) -> np.ndarray:
    """Expert popularity for the skewed workload (float64, sums to 1)."""
    ranks = np.empty(num_experts, dtype=np.float64)
    ranks[rng.permutation(num_experts)] = np.arange(1, num_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    if n_empty > 0:
        empty = {0, num_experts - 1}
        others = [e for e in rng.permutation(num_experts).tolist() if e not in empty]
        empty.update(others[: max(0, n_empty - len(empty))])
        p[sorted(empty)] = 0.0
    return p / p.sum()


def make_routing(w: MoEWorkload, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """(topk_ids int32 [N, topk], topk_weights float32 [N, topk])."""
    st = _streams(seed)
    rng, wrng = st["routing"], st["weights"]
    n, e, k = w.num_tokens, w.num_experts, w.topk
    if w.routing == "uniform":
        keys = rng.random((n, e))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :k]
        weights = _softmax_rows(wrng.standard_normal((n, k)))
    elif w.routing == "softmax_topk":
        probs = _softmax_rows(rng.standard_normal((n, e)))
        ids = np.argsort(-probs, axis=1, kind="stable")[:, :k]
        chosen = np.take_along_axis(probs, ids, axis=1)
        weights = chosen / chosen.sum(axis=1, keepdims=True)
    elif w.routing == "zipf":
        p = zipf_popularity(e, w.zipf_s, w.zipf_empty, rng)
        with np.errstate(divide="ignore"):
            race = rng.exponential(1.0, size=(n, e)) / p[None, :]
        ids = np.argsort(race, axis=1, kind="stable")[:, :k]
        weights = _softmax_rows(wrng.standard_normal((n, k)))
    else:
        raise ValueError(w.routing)
    return np.ascontiguousarray(ids, dtype=np.int32), np.ascontiguousarray(weights, dtype=np.float32)


def _randn(shape, seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def quantize_fp8_per_token(x):
    """fp32 [N, H] torch tensor -> (uint8 codes [N, H], float32 scale [N])."""
    import torch

    amax = x.abs().amax(dim=1)
    scale = amax / FP8_E4M3_MAX
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (x / scale[:, None]).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.to(torch.float32)


def make_hidden(w: MoEWorkload, seed: int = 0, device="cpu"):
    """(hidden_states [N, H] torch tensor of the workload type, token_scale [N] or None).

    fp8 activations come back as uint8 codes with a float32 per-token scale.
    """
    import torch

    st = _streams(seed)
    x = _randn((w.num_tokens, w.hidden_size), st["hidden_seed"], device)
    if w.hidden_dtype == "f32":
        return x, None
    if w.hidden_dtype == "bf16":
        return x.to(torch.bfloat16), None
    if w.hidden_dtype == "fp8_e4m3":
        return quantize_fp8_per_token(x)
    raise ValueError(w.hidden_dtype)


def make_expert_output(w: MoEWorkload, seed: int = 0, device="cpu"):
    """Expanded expert output Y [N*topk, H] (permuted order) of the output type."""
    import torch

    st = _streams(seed)
    y = _randn((w.num_rows, w.hidden_size), st["output_seed"], device)
    if w.output_dtype == "f32":
        return y
    if w.output_dtype == "bf16":
        return y.to(torch.bfloat16)
    raise ValueError(w.output_dtype)


def make_all(w: MoEWorkload, seed: int = 0, device="cpu") -> dict:
    """Every input of one permute + unpermute pass, on ``device``."""
    import torch

    ids, weights = make_routing(w, seed)
    hidden, scale = make_hidden(w, seed, device)
    y = make_expert_output(w, seed, device)
    return {
        "workload": w,
        "topk_ids": torch.from_numpy(ids).to(device),
        "topk_weights": torch.from_numpy(weights).to(device),
        "hidden_states": hidden,
        "token_scale": scale,
        "expert_output": y,
    }
