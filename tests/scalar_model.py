"""A second, scalar implementation of the decoder for brute-force pins.

Pure Python (lists, loops and `math`), no numpy: it shares nothing with the
numpy oracle.  Written directly from the steps of "Dentro de un LLM:
Inferencia en Python puro para Qwen3-0.6B en MLX" (Pasos 2 to 8), for tiny
shapes only.  Attention here materialises every score row and applies the
causal rule by adding -1e9 to scores of future keys, the way the page's listing
masks, instead of excluding them as the oracle does.

bf16 mode: the activations that feed a matrix product are rounded to bf16 at
the points the bf16 model fixes (each RMSNorm output including the final one,
the queries and keys after QK-Norm and RoPE, the values, the merged attention
output, the SwiGLU product), each by rounding the float64 value to the nearest
float32 (the `struct` module's conversion) and that to the nearest bf16, both
ties to even; the second step is written here on the integer bits.
"""
import math
import struct


class Bf16Rounder:
    """Nearest-even rounding of a float64 to bf16 through float32.

    `closest` records, over every value rounded, the smallest relative
    distance between the float64 value and a point where the result of the
    two roundings changes (a bf16 midpoint, or half a float32 step either side
    of it, where the float32 value lands on the midpoint), so a caller can
    tell whether a tiny difference of arithmetic order elsewhere could have
    flipped a rounding."""

    def __init__(self):
        self.closest = math.inf

    @staticmethod
    def _f32(bits: int) -> float:
        return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]

    def __call__(self, v: float) -> float:
        (b,) = struct.unpack("<I", struct.pack("<f", v))   # float64 -> float32, nearest even
        upper, low = b >> 16, b & 0xFFFF
        mid_bits = (upper << 16) | 0x8000
        mid = self._f32(mid_bits)
        half = abs(self._f32(mid_bits + 1) - mid) / 2
        if v != 0.0:
            for edge in (mid - half, mid, mid + half):
                self.closest = min(self.closest, abs(v - edge) / abs(v))
        if low > 0x8000 or (low == 0x8000 and (upper & 1)):
            upper += 1
        return self._f32(upper << 16)

    def vec(self, xs):
        return [self(v) for v in xs]


def _matvec(W, x):
    return [sum(W[o][i] * x[i] for i in range(len(x))) for o in range(len(W))]


def _rmsnorm(x, w, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * w[i] for i in range(len(x))]


def _rope(u, pos, theta):
    half = len(u) // 2
    out = [0.0] * len(u)
    for i in range(half):
        ang = pos * (1.0 / theta ** (i / half))
        c, s = math.cos(ang), math.sin(ang)
        out[i] = u[i] * c - u[i + half] * s
        out[i + half] = u[i] * s + u[i + half] * c
    return out


def scalar_forward_all(d, W, ids, rounder=None):
    """Logits for every position of one prompt processed from an empty cache.

    `rounder` (a Bf16Rounder) turns on the bf16 mode."""
    R = rounder.vec if rounder is not None else (lambda xs: xs)
    L = lambda name: W[name].tolist()
    D = d.head_dim
    group = d.n_q_heads // d.n_kv_heads
    E = L("model.embed_tokens.weight")
    xs = [list(E[t]) for t in ids]
    T = len(ids)
    for layer in range(d.n_layers):
        p = f"model.layers.{layer}"
        wq, wk, wv, wo = (L(f"{p}.self_attn.{n}_proj.weight") for n in "qkvo")
        qn, kn = L(f"{p}.self_attn.q_norm.weight"), L(f"{p}.self_attn.k_norm.weight")
        qs, ks, vs = [], [], []
        for t in range(T):
            h = R(_rmsnorm(xs[t], L(f"{p}.input_layernorm.weight"), d.rms_eps))
            q, k, v = _matvec(wq, h), _matvec(wk, h), _matvec(wv, h)
            qs.append([R(_rope(_rmsnorm(q[a * D:(a + 1) * D], qn, d.rms_eps), t, d.rope_theta))
                       for a in range(d.n_q_heads)])
            ks.append([R(_rope(_rmsnorm(k[a * D:(a + 1) * D], kn, d.rms_eps), t, d.rope_theta))
                       for a in range(d.n_kv_heads)])
            vs.append([R(v[a * D:(a + 1) * D]) for a in range(d.n_kv_heads)])
        new_x = []
        for t in range(T):
            merged = []
            for hq in range(d.n_q_heads):
                g = hq // group
                sc = []
                for j in range(T):
                    s = sum(qs[t][hq][i] * ks[j][g][i] for i in range(D)) / math.sqrt(D)
                    if j > t:
                        s += -1e9
                    sc.append(s)
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                z = sum(e)
                merged += [sum(e[j] / z * vs[j][g][i] for j in range(T)) for i in range(D)]
            a = _matvec(wo, R(merged))
            x1 = [xs[t][i] + a[i] for i in range(d.hidden)]
            h2 = R(_rmsnorm(x1, L(f"{p}.post_attention_layernorm.weight"), d.rms_eps))
            gt = _matvec(L(f"{p}.mlp.gate_proj.weight"), h2)
            up = _matvec(L(f"{p}.mlp.up_proj.weight"), h2)
            mm = R([gt[i] * (1.0 / (1.0 + math.exp(-gt[i]))) * up[i] for i in range(d.ffn)])
            dn = _matvec(L(f"{p}.mlp.down_proj.weight"), mm)
            new_x.append([x1[i] + dn[i] for i in range(d.hidden)])
        xs = new_x
    wf = L("model.norm.weight")
    head = L("lm_head.weight") if "lm_head.weight" in W else E
    return [_matvec(head, R(_rmsnorm(xs[t], wf, d.rms_eps))) for t in range(T)]
