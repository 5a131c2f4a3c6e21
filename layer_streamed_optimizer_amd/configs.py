"""The five workloads: block shapes, parameter counts and hyper-parameters.

Shapes come from the pages:
 * TinyLlama-1.1B (Cloudera community LoRA fine-tuning article, "The full
   memory picture"): 22 layers, hidden 2048, 32 heads, 4 KV heads, FFN 5632,
   vocabulary 32000; LoRA rank 8 on q, k, v, o, gate, up, down of every layer.
 * LLaMA-7B (Transformer Training 09: Memory deck): 32 layers, hidden 4096,
   32 heads, SwiGLU FFN 11008, vocabulary 32000, untied head, RMSNorm;
   6,738,415,616 parameters.
 * A 70B-shaped slice for layer streaming: hidden 8192, 64 heads, 8 KV heads
   of dim 128, SwiGLU FFN 28672, 16 layers.
Values are synthetic (synth package); only the shapes are the models'.
"""
from __future__ import annotations

from dataclasses import dataclass, field

PAGE = 4096          # block sub-arrays start on 4 KB boundaries
TILE = 8192          # elements per tile of the tiled state layout

LR, BETA1, BETA2, EPS = 1e-3, 0.9, 0.999, 1e-8
MASTER_SIGMA, GRAD_SIGMA, LORA_A_SIGMA = 0.02, 1e-3, 1.0 / 8.0


def align(x: int, a: int = PAGE) -> int:
    return (x + a - 1) // a * a


@dataclass(frozen=True)
class BlockSpec:
    name: str
    n: int
    init: str = "normal"         # "normal" (sigma master_sigma), "lora_a", "zero"


@dataclass
class Workload:
    key: str
    title: str
    blocks: list[BlockSpec]
    steps: int
    streamed: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def params(self) -> int:
        return sum(b.n for b in self.blocks)


def decoder_layer(hidden: int, heads: int, kv_heads: int, head_dim: int, ffn: int) -> list[tuple[str, int]]:
    """Parameter tensors of one LLaMA-style decoder layer (no biases)."""
    q = hidden * heads * head_dim
    kv = hidden * kv_heads * head_dim
    return [("q_proj", q), ("k_proj", kv), ("v_proj", kv), ("o_proj", heads * head_dim * hidden),
            ("gate_proj", ffn * hidden), ("up_proj", ffn * hidden), ("down_proj", hidden * ffn),
            ("input_norm", hidden), ("post_attn_norm", hidden)]


def layer_params(**shape) -> int:
    return sum(n for _, n in decoder_layer(**shape))


TINYLLAMA = dict(hidden=2048, heads=32, kv_heads=4, head_dim=64, ffn=5632)
LLAMA7B = dict(hidden=4096, heads=32, kv_heads=32, head_dim=128, ffn=11008)
LLAMA70B = dict(hidden=8192, heads=64, kv_heads=8, head_dim=128, ffn=28672)
VOCAB = 32000


def c0_flat() -> Workload:
    return Workload("c0", "one flat 1024x1024 block, device-resident",
                    [BlockSpec("w", 1024 * 1024)], steps=10)


def c1_tinyllama() -> Workload:
    """22 contiguous layer blocks + embedding + untied head + final norm.
    The final RMSNorm (2048) is counted: it makes the 1.10B of the page."""
    h = TINYLLAMA["hidden"]
    per = layer_params(**TINYLLAMA)
    blocks = [BlockSpec("embed", VOCAB * h)]
    blocks += [BlockSpec(f"layer{i}", per) for i in range(22)]
    blocks += [BlockSpec("final_norm", h), BlockSpec("lm_head", VOCAB * h)]
    return Workload("c1", "TinyLlama-1.1B shape, device-resident", blocks, steps=10,
                    notes={"layer_params": per})


def lora_targets(hidden: int, heads: int, kv_heads: int, head_dim: int, ffn: int) -> list[tuple[str, int, int]]:
    """(name, d_in, d_out) of the seven LoRA targets of one layer."""
    q = heads * head_dim
    kv = kv_heads * head_dim
    return [("q", hidden, q), ("k", hidden, kv), ("v", hidden, kv), ("o", q, hidden),
            ("gate", hidden, ffn), ("up", hidden, ffn), ("down", ffn, hidden)]


def c2_lora(rank: int = 8) -> Workload:
    """Rank-r A (r x d_in, N(0, 1/8)) and B (d_out x r, zero) per target:
    14 tensors per layer, 308 ragged tensors in all."""
    blocks = []
    for layer in range(22):
        for name, d_in, d_out in lora_targets(**TINYLLAMA):
            blocks.append(BlockSpec(f"l{layer}.{name}.A", rank * d_in, "lora_a"))
            blocks.append(BlockSpec(f"l{layer}.{name}.B", d_out * rank, "zero"))
    return Workload("c2", "LoRA r=8 adapters on TinyLlama, 308 ragged tensors", blocks, steps=100)


def c3_llama7b() -> Workload:
    h = LLAMA7B["hidden"]
    per = layer_params(**LLAMA7B)
    blocks = [BlockSpec("embed", VOCAB * h)]
    blocks += [BlockSpec(f"layer{i}", per) for i in range(32)]
    blocks += [BlockSpec("final_norm", h), BlockSpec("lm_head", VOCAB * h)]
    return Workload("c3", "LLaMA-7B shape, device-resident", blocks, steps=5,
                    notes={"layer_params": per})


def c4_streamed70b(layers: int = 16) -> Workload:
    per = layer_params(**LLAMA70B)
    blocks = [BlockSpec(f"layer{i}", per) for i in range(layers)]
    return Workload("c4", "70B-shaped slice, layer-streamed from host memory", blocks,
                    steps=3, streamed=True, notes={"layer_params": per})


WORKLOADS = {"c0": c0_flat, "c1": c1_tinyllama, "c2": c2_lora, "c3": c3_llama7b, "c4": c4_streamed70b}
STREAM_ID = {"c0": 0, "c1": 1, "c2": 2, "c3": 3, "c4": 4}   # RNG stream per workload


def get(key: str) -> Workload:
    return WORKLOADS[key]()


# ------------------------------------------------------------ HBM layout

def tiled_state_bytes(n: int) -> int:
    """Bytes of the tiled [master | m | v] state of n parameters."""
    return 12 * TILE * ((n + TILE - 1) // TILE)


@dataclass
class ResidentLayout:
    """Byte offsets of every array in three device arenas.

    state arena:  per block [master | m | v], FP32, each 4 KB aligned
                  (tiled: one region per block, master/m/v interleaved per
                  TILE elements; off_m / off_v then equal off_master)
    grad arena:   per block BF16 gradients (FP32 with grad_f32), 4 KB aligned
    weight arena: per block BF16 re-cast weights, 4 KB aligned
    A block's state is contiguous (the same shape as a streamed host block),
    so a layer can move between host and HBM as one copy.
    """
    sizes: list[int]
    tiled: bool = False
    grad_f32: bool = False
    off_master: list[int] = field(default_factory=list)
    off_m: list[int] = field(default_factory=list)
    off_v: list[int] = field(default_factory=list)
    off_grad: list[int] = field(default_factory=list)
    off_weight: list[int] = field(default_factory=list)
    state_bytes: int = 0
    grad_bytes: int = 0
    weight_bytes: int = 0

    def __post_init__(self):
        s = g = w = 0
        for n in self.sizes:
            if self.tiled:
                self.off_master.append(s)
                self.off_m.append(s)
                self.off_v.append(s)
                s += align(tiled_state_bytes(n))
            else:
                a = align(4 * n)
                self.off_master.append(s)
                self.off_m.append(s + a)
                self.off_v.append(s + 2 * a)
                s += 3 * a
            self.off_grad.append(g)
            g += align((4 if self.grad_f32 else 2) * n)
            self.off_weight.append(w)
            w += align(2 * n)
        self.state_bytes, self.grad_bytes, self.weight_bytes = s, g, w


@dataclass
class BlockArena:
    """Byte offsets of every array in one device arena, block after block:
    [state | BF16 weights | gradient set 0 | ... | gradient set k-1], each
    array 4 KB aligned (state as in ResidentLayout: tiled, or planar
    [master | m | v]).

    The arrays one block's update streams together sit next to each other.
    Measured on MI355X (c3, LLaMA-7B), the update then runs at the same rate
    wherever the arena lands in HBM (28.78-28.85 ms at 12 placements), where
    three separate regions (all states, all weights, all gradients) run at
    28.37-29.22 ms depending on placement.  It is for calls that stream HBM:
    a cache-sized call (c2, 308 small tensors) spread over per-block groups
    touches ten times the pages and ran slower (34.0 against 30.1 us) than
    in compact regions (ResidentLayout).
    """
    sizes: list[int]
    tiled: bool = False
    grad_f32: bool = False
    grad_sets: int = 1
    off_master: list[int] = field(default_factory=list)
    off_m: list[int] = field(default_factory=list)
    off_v: list[int] = field(default_factory=list)
    off_weight: list[int] = field(default_factory=list)
    off_grad: list[list[int]] = field(default_factory=list)   # [set][block]
    total_bytes: int = 0
    state_bytes: int = 0     # sums over blocks (what each kind of array takes)
    grad_bytes: int = 0      # one gradient set
    weight_bytes: int = 0

    def __post_init__(self):
        if self.grad_sets < 1:
            raise ValueError("grad_sets must be >= 1")
        self.off_grad = [[] for _ in range(self.grad_sets)]
        pos = 0
        for n in self.sizes:
            if self.tiled:
                st = align(tiled_state_bytes(n))
                self.off_master.append(pos)
                self.off_m.append(pos)
                self.off_v.append(pos)
            else:
                a = align(4 * n)
                st = 3 * a
                self.off_master.append(pos)
                self.off_m.append(pos + a)
                self.off_v.append(pos + 2 * a)
            pos += st
            self.state_bytes += st
            wb = align(2 * n)
            self.off_weight.append(pos)
            pos += wb
            self.weight_bytes += wb
            gb = align((4 if self.grad_f32 else 2) * n)
            for r in range(self.grad_sets):
                self.off_grad[r].append(pos)
                pos += gb
            self.grad_bytes += gb
        self.total_bytes = pos


def host_layer_layout(n: int, tiled: bool = False) -> tuple[int, int, int, int]:
    """(off_master, off_m, off_v, bytes) of one streamed host block:
    [master | m | v] with 4 KB-aligned sub-arrays, or one tiled region."""
    if tiled:
        b = align(tiled_state_bytes(n))
        return 0, 0, 0, b
    a = align(4 * n)
    return 0, a, 2 * a, 3 * a
