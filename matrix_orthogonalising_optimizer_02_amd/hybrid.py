"""Hybrid optimizer: Muon for the 2-D weights inside transformer blocks, AdamW for the rest.

"Scaling Muon for Diffusion Transformers" (setup paragraph) applies Muon only to the
2-D weights of the transformer blocks, about 99% of the trainable parameters, and keeps
biases, normalisation parameters and every parameter outside the blocks on an
auxiliary AdamW group (lr 1e-4). "Muon is Scalable for LLM Training" (Sec. 2.2,
matching-update-RMS paragraph) pairs the two the same way and lets them share the
weight decay. Both halves run in libmuon_rocm.so: muon_step for the Muon group (one
launch sequence per step for all of its matrices) and adamw_step for the AdamW group.

`dit_parameter_list` names and shapes the parameters of a double-stream (image and
text) diffusion transformer, whose block matrices are the pages' DiT shapes: qkv
[3H, H], proj [H, H], MLP up [4H, H] and down [H, 4H], adaLN modulation [6H, H].
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from . import binding as B

BLOCK_PREFIX = "blocks."

# Scales of the pages' model family (1.3B, 4B, 9B, 15B), read as hidden size and depth
# of a double-stream backbone whose block holds 2 x 18 H^2 matrix weights.
DIT_SCALES = {
    "1.3B": (2048, 9),
    "4B": (3072, 12),
    "9B": (4096, 15),
    "15B": (5120, 16),
}


def goes_to_muon(name: str, shape: Sequence[int]) -> bool:
    """2-D parameters inside a transformer block go to Muon; everything else to AdamW."""
    return len(shape) == 2 and name.startswith(BLOCK_PREFIX)


def split_param_groups(named_shapes) -> Tuple[List[str], List[str]]:
    """(Muon names, AdamW names) for an iterable of (name, shape), order preserved."""
    muon, adamw = [], []
    for name, shape in named_shapes:
        (muon if goes_to_muon(name, tuple(shape)) else adamw).append(name)
    return muon, adamw


def dit_parameter_list(hidden: int, depth: int, head_dim: int = 128, latent_channels: int = 16,
                       patch: int = 2, text_dim: int = 4096, pooled_dim: int = 2048,
                       freq_dim: int = 256) -> List[Tuple[str, Tuple[int, ...]]]:
    """(name, shape) of every trainable parameter of a double-stream DiT.

    Per block and stream: attention qkv and output projection, q/k RMSNorm weights,
    a 4x MLP and the adaLN modulation, each linear with a bias. Outside the blocks:
    patch and text embedders, the timestep and pooled-text embedders, and the final
    adaLN + projection layer (latent channels x patch^2 outputs).
    """
    h = hidden
    out_dim = latent_channels * patch * patch
    params: List[Tuple[str, Tuple[int, ...]]] = []

    def linear(name, rows, cols):
        params.append((f"{name}.weight", (rows, cols)))
        params.append((f"{name}.bias", (rows,)))

    linear("x_embedder", h, out_dim)
    linear("context_embedder", h, text_dim)
    linear("time_embed.fc1", h, freq_dim)
    linear("time_embed.fc2", h, h)
    linear("pooled_embed.fc1", h, pooled_dim)
    for i in range(depth):
        for stream in ("img", "txt"):
            p = f"{BLOCK_PREFIX}{i}.{stream}"
            linear(f"{p}.attn.qkv", 3 * h, h)
            params.append((f"{p}.attn.q_norm.weight", (head_dim,)))
            params.append((f"{p}.attn.k_norm.weight", (head_dim,)))
            linear(f"{p}.attn.proj", h, h)
            linear(f"{p}.mlp.up", 4 * h, h)
            linear(f"{p}.mlp.down", h, 4 * h)
            linear(f"{p}.mod", 6 * h, h)
    linear("final_layer.mod", 2 * h, h)
    linear("final_layer.linear", out_dim, h)
    return params


def count_params(named_shapes) -> Tuple[int, int]:
    """(Muon elements, AdamW elements)."""
    mu = ad = 0
    for name, shape in named_shapes:
        n = 1
        for d in shape:
            n *= int(d)
        if goes_to_muon(name, tuple(shape)):
            mu += n
        else:
            ad += n
    return mu, ad


class HybridOptimizer:
    """Periodic Row-wise Muon on the block matrices plus AdamW on the other parameters.

    named_params: mapping name -> fp32 CUDA tensor (contiguous). step(grads) takes a
    mapping with the same names and advances every parameter by one step; both groups
    share the 0-based step counter (Muon's refresh schedule, AdamW's bias correction).
    """

    def __init__(self, named_params: Dict[str, "object"], muon_hp: Optional[B.MuonHParams] = None,
                 adamw_hp: Optional[B.AdamWHParams] = None):
        import torch
        self.names = list(named_params)
        shapes = [(n, tuple(named_params[n].shape)) for n in self.names]
        self.muon_names, self.adamw_names = split_param_groups(shapes)
        self.params = named_params
        self.muon_hp = muon_hp or B.default_hparams()
        self.adamw_hp = adamw_hp or B.adamw_default_hparams()
        self.momenta = {n: torch.zeros_like(named_params[n]) for n in self.muon_names}
        self.exp_avg = {n: torch.zeros_like(named_params[n]) for n in self.adamw_names}
        self.exp_avg_sq = {n: torch.zeros_like(named_params[n]) for n in self.adamw_names}
        dev = next(iter(named_params.values())).device if named_params else "cuda"
        self.workspace = B.make_workspace([tuple(named_params[n].shape) for n in self.muon_names], dev) \
            if self.muon_names else None
        self._adamw = None  # descriptor array, built at the first step
        self.step_count = 0

    def step(self, grads: Dict[str, "object"], stream=None, update_rms=None):
        if self.muon_names:
            B.muon_step([self.params[n] for n in self.muon_names], [self.momenta[n] for n in self.muon_names],
                        [grads[n] for n in self.muon_names], self.step_count, self.muon_hp, self.workspace,
                        stream, update_rms)
        if self.adamw_names:
            g = [grads[n] for n in self.adamw_names]
            if self._adamw is None:
                self._adamw = B.AdamWGroup([self.params[n] for n in self.adamw_names], g,
                                           [self.exp_avg[n] for n in self.adamw_names],
                                           [self.exp_avg_sq[n] for n in self.adamw_names], self.adamw_hp)
                self._adamw.step(self.step_count, stream)
            else:
                same = all(a is b for a, b in zip(g, self._adamw.tensors[1]))
                self._adamw.step(self.step_count, stream, None if same else g)
        self.step_count += 1

    def state_dict(self):
        return {"step": self.step_count,
                "momenta": {n: t.clone() for n, t in self.momenta.items()},
                "exp_avg": {n: t.clone() for n, t in self.exp_avg.items()},
                "exp_avg_sq": {n: t.clone() for n, t in self.exp_avg_sq.items()}}

    def load_state_dict(self, state):
        self.step_count = int(state["step"])
        for key, dst in (("momenta", self.momenta), ("exp_avg", self.exp_avg), ("exp_avg_sq", self.exp_avg_sq)):
            for n, t in dst.items():
                t.copy_(state[key][n])
