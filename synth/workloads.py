"""Model shapes and run protocols of the synthetic decode workloads.

Five Llama-style decoders, batch 1:
  tiny      2 layers, hidden 256, 4 q / 2 kv heads, head_dim 64, FFN 688,
            vocab 4096, theta 1e4; 16-token prompt, 32 decode steps
  1b        16 layers, hidden 2048, 32 q / 8 kv heads, head_dim 64, FFN 8192,
            vocab 128256, tied embeddings; 128-token prompt, 128 decode steps
  8b        32 layers, hidden 4096, 32 q / 8 kv heads, head_dim 128,
            FFN 14336, vocab 128256, theta 5e5; 1024-token prompt, 256 steps
  8b_int8   8b with int8 per-output-row weights (fp32 scales), bf16
            activations at every projection input
  8b_int8_a32  8b_int8's weights with fp32 projection inputs (a check of the
            int8 path at the plain parity bar; not a benchmark workload)
  8b_int4   8b with int4 weights in groups of 128 (fp16 scale + zero),
            8192-token prompt, 128 decode steps

Canonical tensors follow the Hugging Face Linear layout [out][in]; ids are
  0                   token embedding  [vocab][hidden]
  1 + 9*l + k         layer l: k = 0 attn_norm, 1 wq, 2 wk, 3 wv, 4 wo,
                      5 mlp_norm, 6 w_gate, 7 w_up, 8 w_down
  1 + 9*L             final_norm
  2 + 9*L             lm_head (absent when embeddings are tied)
"""
from dataclasses import dataclass, replace

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    tied: bool = False
    wfmt: str = "bf16"          # "bf16" | "int8" | "int4"
    act_bf16: bool = False      # projection inputs rounded to bf16
    prompt_len: int = 16
    decode_steps: int = 32
    max_ctx: int = 64

    def with_(self, **kw):
        return replace(self, **kw)


def _ctx(p, s):
    n = p + s
    return (n + 63) // 64 * 64


CONFIGS = {
    "tiny": Workload("tiny", 2, 256, 4, 2, 64, 688, 4096, 1e-5, 10000.0, False, "bf16", False,
                     16, 32, _ctx(16, 32)),
    "1b": Workload("1b", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5, 10000.0, True, "bf16", False,
                   128, 128, _ctx(128, 128)),
    "8b": Workload("8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, False, "bf16",
                   False, 1024, 256, _ctx(1024, 256)),
    "8b_int8": Workload("8b_int8", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, False,
                        "int8", True, 1024, 256, _ctx(1024, 256)),
    # the same int8 weights with fp32 projection inputs (W8A32): the int8
    # GEMV held to the plain parity bar, without the bf16 activation roundings
    "8b_int8_a32": Workload("8b_int8_a32", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, False,
                            "int8", False, 1024, 256, _ctx(1024, 256)),
    "8b_int4": Workload("8b_int4", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, False,
                        "int4", False, 8192, 128, _ctx(8192, 128)),
}


def get(name):
    return CONFIGS[name]


def tensor_shape(wl, name):
    H, F, V = wl.hidden, wl.ffn, wl.vocab
    q, kv = wl.n_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim
    return {
        "embed": (V, H), "final_norm": (H,), "lm_head": (V, H),
        "attn_norm": (H,), "mlp_norm": (H,),
        "wq": (q, H), "wk": (kv, H), "wv": (kv, H), "wo": (H, q),
        "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
    }[name]


def canonical_tensors(wl):
    """[(tensor id, name, shape)] in canonical order."""
    out = [(0, "embed", tensor_shape(wl, "embed"))]
    for l in range(wl.n_layers):
        for k, nm in enumerate(LAYER_TENSORS):
            out.append((1 + 9 * l + k, nm, tensor_shape(wl, nm)))
    out.append((1 + 9 * wl.n_layers, "final_norm", tensor_shape(wl, "final_norm")))
    if not wl.tied:
        out.append((2 + 9 * wl.n_layers, "lm_head", tensor_shape(wl, "lm_head")))
    return out


def n_canonical(wl):
    """Size of the canonical id space (lm_head slot included even if tied)."""
    return 3 + 9 * wl.n_layers
