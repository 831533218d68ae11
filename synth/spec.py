"""Model shapes and the ordered weight-tensor list of the Moshi frame step.

The order below is the layout contract of the weight pointer array handed to
both the oracle and the HIP library (each indexes it with code of its own).
Every tensor is row-major; a projection matrix ``[N, K]`` maps a K-vector to an
N-vector (row n is output n).

Shapes follow the architecture notes of the pages:
* temporal transformer 4096-d / 32 layers / 32 heads, sliding window of 3000
  frames (vLLM-Omni PersonaPlex recipe, "Architecture");
* depformer 1024-d / 6 layers / 16 heads, one substep per codebook, with
  per-substep linears (mobius PR #368, "P2 - Moshi LM");
* a 17-row token column: text, 8 agent and 8 user audio codebooks (recipe,
  "Architecture"); text vocabulary 32000, audio card 2048.

Tensor ids (the ``tensor`` argument of the seeded draws) are list positions.
"""
from dataclasses import dataclass, asdict, replace


@dataclass(frozen=True)
class ModelShape:
    dim: int
    n_layers: int
    n_heads: int
    ffn: int
    window: int
    dep_dim: int
    dep_layers: int
    dep_heads: int
    dep_ffn: int
    n_substeps: int
    text_vocab: int
    audio_card: int
    rope_theta: float = 1e4
    norm_eps: float = 1e-8
    dtype: str = "bf16"          # "bf16" or "f32"
    mask_oldest: bool = False    # window reading flag (attend W-1 keys once full)
    dep_q: int = 0               # depformer substeps run per frame (0 = all)
    dep_final_norm: bool = False # RMSNorm (gain dep.out_norm) before each depformer head
    dep_ref_ring: bool = False   # mask substep entry 0 at the last substep run

    @property
    def head_dim(self):
        return self.dim // self.n_heads

    @property
    def dep_head_dim(self):
        return self.dep_dim // self.dep_heads

    @property
    def n_channels(self):
        return 1 + self.n_substeps

    @property
    def dep_steps(self):
        return self.dep_q if 0 < self.dep_q < self.n_substeps else self.n_substeps

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4

    def asdict(self):
        return asdict(self)

    def replace(self, **kw):
        return replace(self, **kw)


# The PersonaPlex-shape model (temporal + depformer), bf16.
PERSONAPLEX = ModelShape(dim=4096, n_layers=32, n_heads=32, ffn=11264, window=3000,
                         dep_dim=1024, dep_layers=6, dep_heads=16, dep_ffn=2816, n_substeps=16,
                         text_vocab=32000, audio_card=2048, dtype="bf16")

# The tiny fp32 model.
TINY = ModelShape(dim=256, n_layers=2, n_heads=4, ffn=704, window=64,
                  dep_dim=128, dep_layers=2, dep_heads=4, dep_ffn=352, n_substeps=16,
                  text_vocab=32000, audio_card=2048, dtype="f32")

# A small bf16 model with ragged sizes (rows, K and window not multiples of the
# kernel tiles), used by parity tests that must span several tiles and a tail.
RAGGED = ModelShape(dim=384, n_layers=2, n_heads=3, ffn=1000, window=37,
                    dep_dim=192, dep_layers=2, dep_heads=3, dep_ffn=520, n_substeps=16,
                    text_vocab=1000, audio_card=300, dtype="bf16")


def tensor_list(m: ModelShape):
    """Ordered list of (name, shape, kind); kind is "normal" or "gain"."""
    D, L, F = m.dim, m.n_layers, m.ffn
    Dd, Ld, Fd, S = m.dep_dim, m.dep_layers, m.dep_ffn, m.n_substeps
    Vt, Va = m.text_vocab, m.audio_card
    t = []
    # 17-channel input embeddings: one row per code plus one "initial token" row.
    t.append(("emb.text", (Vt + 1, D), "normal"))
    for k in range(S):
        t.append((f"emb.audio.{k}", (Va + 1, D), "normal"))
    for l in range(L):
        t.append((f"layer.{l}.attn_norm", (D,), "gain"))
        t.append((f"layer.{l}.qkv", (3 * D, D), "normal"))      # rows: q | k | v
        t.append((f"layer.{l}.o", (D, D), "normal"))
        t.append((f"layer.{l}.mlp_norm", (D,), "gain"))
        t.append((f"layer.{l}.gate_up", (2 * F, D), "normal"))  # rows: gate | up
        t.append((f"layer.{l}.down", (D, F), "normal"))
    t.append(("out_norm", (D,), "gain"))
    t.append(("text_head", (Vt, D), "normal"))
    for s in range(S):
        t.append((f"dep.in.{s}", (Dd, D), "normal"))
    t.append(("dep.emb.0", (Vt + 1, Dd), "normal"))
    for s in range(1, S):
        t.append((f"dep.emb.{s}", (Va + 1, Dd), "normal"))
    for l in range(Ld):
        t.append((f"dep.layer.{l}.attn_norm", (Dd,), "gain"))
        t.append((f"dep.layer.{l}.mlp_norm", (Dd,), "gain"))
    for s in range(S):
        for l in range(Ld):
            t.append((f"dep.{s}.layer.{l}.qkv", (3 * Dd, Dd), "normal"))
            t.append((f"dep.{s}.layer.{l}.o", (Dd, Dd), "normal"))
            t.append((f"dep.{s}.layer.{l}.gate_up", (2 * Fd, Dd), "normal"))
            t.append((f"dep.{s}.layer.{l}.down", (Dd, Fd), "normal"))
    for s in range(S):
        t.append((f"dep.head.{s}", (Va, Dd), "normal"))
    if m.dep_final_norm:
        t.append(("dep.out_norm", (Dd,), "gain"))
    return t


def n_tensors(m: ModelShape) -> int:
    return len(tensor_list(m))


def weight_bytes(m: ModelShape) -> int:
    tot = 0
    for _, shp, _ in tensor_list(m):
        n = 1
        for s in shp:
            n *= s
        tot += n * m.elem_bytes
    return tot


def kv_bytes_per_frame(m: ModelShape) -> int:
    """Bytes of temporal K and V that one frame adds to a session's cache."""
    return 2 * m.n_layers * m.dim * m.elem_bytes
