"""Seeded synthetic inputs for the five CSA2 workloads.

This module draws random tensors and nothing else: it holds none of the
path's arithmetic (no pooling, quantisation, scoring, selection or
attention).  Both the HIP path and the fp64 oracle read the tensors it
returns -- large ones are drawn on the device and the oracle receives host
copies of the slices it checks.

Shapes and distributions follow the workload statements: 512-d latents and
compression logits N(0, 1) in bf16, an indexer-K projection N(0, 1/512) in
bf16 stored [128, 512] (output dim x input channel), indexer queries
32 x 128 N(0, 1) bf16 with head weights U(0, 1) fp32, attention queries
64 x 512 N(0, 1)/sqrt(512) bf16, and FP8 E4M3FN SWA rows with one fp32 scale
per row (a N(0, 1) latent divided by max|row| / 448 and converted by torch's
own float8_e4m3fn cast).

Every tensor has its own torch.Generator seeded from (workload seed, tensor
tag, layer); workload c uses seed c.
"""

from dataclasses import dataclass, field
import math

import torch

TAGS = {"h": 1, "z": 2, "w_ik": 3, "q_idx": 4, "w": 5, "q_attn": 6, "swa": 7}


def _gen(seed, tag, layer, device):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + TAGS[tag] * 10_007 + layer * 101) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


@dataclass
class Workload:
    """One of the five configurations.

    name        short name ("c0".."c4")
    B           sequences
    T           raw tokens per sequence
    m           compression ratio (entries = T / m)
    layers      list of layer modes after the cache is built:
                "full", "reindex" or "reuse"
    hierarchical  whether the Full layer builds the 2048 x 8 candidate pool
    prefill     causal prefill (one sequence, one query per entry) instead of
                one decode query per sequence
    q_chunk     prefill queries per chunk (0: all at once)
    draw_device draw the per-layer inputs on the device (large prefills)
    reuse_chunk_inputs  the per-layer queries are drawn for one chunk of
                q_chunk queries and every chunk uses them (and writes its
                outputs into one chunk-sized buffer): at 2^19 queries the
                full-size query and output tensors would not fit in memory,
                and the work of a chunk does not depend on the values
    """
    name: str
    seed: int
    B: int
    T: int
    m: int
    layers: list
    hierarchical: bool = False
    prefill: bool = False
    k: int = 512
    swa: int = 128
    block: int = 8
    n_blocks: int = 2048
    q_chunk: int = 0
    draw_device: bool = False
    reuse_chunk_inputs: bool = False
    note: str = ""

    @property
    def N(self):
        return self.T // self.m

    @property
    def Q(self):
        return self.N if self.prefill else self.B

    @property
    def T_swa(self):
        return self.T if self.prefill else self.swa

    # ------------------------------------------------------------ draws
    def latents(self, device, b0=0, b1=None):
        """h [B, T, 512] bf16 and z (None when m == 1) for sequences b0..b1."""
        b1 = self.B if b1 is None else b1
        hs, zs = [], []
        for b in range(b0, b1):
            hs.append(torch.randn(self.T, 512, dtype=torch.bfloat16, device=device,
                                  generator=_gen(self.seed, "h", b, device)))
            if self.m > 1:
                zs.append(torch.randn(self.T, 512, dtype=torch.bfloat16, device=device,
                                      generator=_gen(self.seed, "z", b, device)))
        h = torch.stack(hs)
        z = torch.stack(zs) if zs else None
        return h, z

    def w_ik(self, device="cpu"):
        g = _gen(self.seed, "w_ik", 0, "cpu")
        w = torch.randn(128, 512, dtype=torch.float32, generator=g) / math.sqrt(512.0)
        return w.to(torch.bfloat16).to(device)

    @property
    def input_rows(self):
        """Rows of the per-layer query tensors (and of the step's outputs)."""
        return self.q_chunk if (self.reuse_chunk_inputs and self.q_chunk) else self.Q

    def layer_inputs(self, layer, device="cpu"):
        """Per-layer queries and SWA rows (drawn on the CPU, then moved)."""
        Q = self.input_rows
        out = {}
        dd = device if self.draw_device else "cpu"
        g = _gen(self.seed, "q_idx", layer, dd)
        out["q_idx"] = torch.randn(Q, 32, 128, dtype=torch.float32, generator=g,
                                   device=dd).to(torch.bfloat16)
        g = _gen(self.seed, "w", layer, dd)
        out["w"] = torch.rand(Q, 32, dtype=torch.float32, generator=g, device=dd)
        g = _gen(self.seed, "q_attn", layer, dd)
        out["q_attn"] = (torch.randn(Q, 64, 512, dtype=torch.float32, generator=g, device=dd)
                         / math.sqrt(512.0)).to(torch.bfloat16)
        nseq = 1 if self.prefill else self.B
        g = _gen(self.seed, "swa", layer, dd)
        lat = torch.randn(nseq, self.T_swa, 512, dtype=torch.float32, generator=g, device=dd)
        scale = lat.abs().amax(dim=2) / 448.0
        codes = (lat / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
        out["swa_codes"] = codes
        out["swa_scale"] = scale.contiguous()
        return {k: v.to(device) for k, v in out.items()}

    # ------------------------------------------------------ query geometry
    def query_geometry(self):
        """Per query: sequence, visible entries, SWA window start / length.

        Decode: one query per sequence sees all N entries and its own
        128-row window.  Prefill (m = 2): query i sits at raw position
        2i + 1, sees entries 0..i (entry j covers raw rows 2j, 2j+1 and is
        complete once row 2j+1 exists) and the SWA rows
        [max(0, 2i+1-127), 2i+1] of the chunk's own FP8 rows."""
        Q = self.Q
        if not self.prefill:
            q_seq = torch.arange(Q, dtype=torch.int32)
            n_vis = torch.full((Q,), self.N, dtype=torch.int64)
            swa_start = torch.zeros(Q, dtype=torch.int64)
            swa_len = torch.full((Q,), self.swa, dtype=torch.int32)
        else:
            i = torch.arange(Q, dtype=torch.int64)
            pos = i * self.m + (self.m - 1)
            q_seq = torch.zeros(Q, dtype=torch.int32)
            n_vis = i + 1
            swa_start = torch.clamp(pos - (self.swa - 1), min=0)
            swa_len = (pos - swa_start + 1).to(torch.int32)
        return dict(q_seq=q_seq, n_vis=n_vis, swa_start=swa_start, swa_len=swa_len)


WORKLOADS = {
    "c0": Workload("c0", 0, B=1, T=2048, m=1, layers=["full"],
                   note="tiny full-layer decode, N=2048"),
    "c1": Workload("c1", 1, B=32, T=65536, m=1, layers=["full"],
                   note="batched full-layer decode, 32 x N=65536"),
    "c2": Workload("c2", 2, B=4, T=1 << 20, m=1,
                   layers=["full", "reindex", "reindex", "reindex", "reindex"], hierarchical=True,
                   note="hierarchical decoder decode at 1M context, batch 4"),
    "c3": Workload("c3", 3, B=1, T=8192, m=2, layers=["full"], prefill=True,
                   note="encoder full-layer prefill chunk, 8192 raw tokens, m=2"),
    "c4": Workload("c4", 4, B=8, T=1 << 20, m=2,
                   layers=["full", "reuse", "reuse", "reuse", "reuse", "reuse"],
                   note="encoder long-context decode with reuse, 1M raw tokens, m=2, batch 8"),
    # long encoder prefill in query chunks: one encoder group (Full + 5 Reuse)
    "p64k": Workload("p64k", 5, B=1, T=1 << 16, m=2,
                     layers=["full", "reuse", "reuse", "reuse", "reuse", "reuse"], prefill=True,
                     q_chunk=4096, draw_device=True,
                     note="encoder group prefill of 65,536 raw tokens (m=2) in 4096-query chunks"),
    "p1m": Workload("p1m", 6, B=1, T=1 << 20, m=2,
                    layers=["full", "reuse", "reuse", "reuse", "reuse", "reuse"], prefill=True,
                    q_chunk=4096, draw_device=True, reuse_chunk_inputs=True,
                    note="encoder group prefill of 1,048,576 raw tokens (m=2) in 4096-query "
                         "chunks, one chunk's queries reused by every chunk"),
}


def scaled(w: Workload, **kw):
    """A copy of a workload with some sizes changed (for small test cases)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)
