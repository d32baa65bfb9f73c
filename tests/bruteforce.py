"""Scalar-loop decoder written straight from the definitions, for pinning the
oracle on tiny shapes.  Pure Python floats (IEEE double) and the math module;
no numpy arithmetic, no code shared with oracle/ or the HIP path.

Block (pre-norm, per token t at position p, caches per layer):
  h = g_a * x / sqrt(mean(x^2) + eps)
  q = Wq h, k = Wk h, v = Wv h            (W is [out][in]: y_i = sum_j W[i][j] x_j)
  rotate pairs (i, i + hd/2) of each q and k head by p * base^(-2i/hd)
  head i attends with KV head i // (H / Hkv) over keys 0..p, scale 1/sqrt(hd)
  sequential: x += Wo o; x += Wd (silu(Wg h2) * (Wu h2)), h2 = norm(x, g_m)
  parallel, delay D: P_l = Wo o + Wd(...)(norm(x_l, g_m)); x_{l+1} = x_l + P_{l-D};
                     the last D partials are added before the final norm
  logits = W_lm (g_f * x / rms(x))
"""
import math


def tolist(a):
    return a.astype("float64").tolist()


def rms(x, g, eps):
    ms = 0.0
    for v in x:
        ms += v * v
    ms /= len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def matvec(W, x):
    out = []
    for row in W:
        s = 0.0
        for j in range(len(x)):
            s += row[j] * x[j]
        out.append(s)
    return out


def rope(u, pos, base):
    hd = len(u)
    half = hd // 2
    out = [0.0] * hd
    for i in range(half):
        th = pos * base ** (-2.0 * i / hd)
        c, s = math.cos(th), math.sin(th)
        out[i] = u[i] * c - u[i + half] * s
        out[i + half] = u[i] * s + u[i + half] * c
    return out


def silu(z):
    return z / (1.0 + math.exp(-z))


def to_half(x):
    """round a Python float to the nearest binary16 value (ties to even)"""
    import struct
    return struct.unpack("<e", struct.pack("<e", x))[0]


class BruteDecoder:
    def __init__(self, cfg, weights, kv_fp16=False):
        self.kv_fp16 = kv_fp16
        self.c = cfg
        self.w = {k: tolist(v) for k, v in weights.items()}
        self.K = [[[] for _ in range(cfg.n_kv_heads)] for _ in range(cfg.n_layers)]
        self.V = [[[] for _ in range(cfg.n_kv_heads)] for _ in range(cfg.n_layers)]

    def lw(self, l, n):
        return self.w[f"layers.{l}.{n}"]

    def attn(self, l, x, pos):
        c = self.c
        hd, H, Hkv = c.head_dim, c.n_heads, c.n_kv_heads
        G = H // Hkv
        h = rms(x, self.lw(l, "attn_norm"), c.rms_eps)
        q = matvec(self.lw(l, "wq"), h)
        k = matvec(self.lw(l, "wk"), h)
        v = matvec(self.lw(l, "wv"), h)
        rnd = to_half if self.kv_fp16 else (lambda t: t)
        for g in range(Hkv):
            self.K[l][g].append([rnd(t) for t in rope(k[g * hd:(g + 1) * hd], pos, c.rope_base)])
            self.V[l][g].append([rnd(t) for t in v[g * hd:(g + 1) * hd]])
        o = []
        for i in range(H):
            qi = rope(q[i * hd:(i + 1) * hd], pos, c.rope_base)
            g = i // G
            keys = self.K[l][g]
            assert len(keys) == pos + 1
            sc = []
            for kj in keys:
                s = 0.0
                for e in range(hd):
                    s += qi[e] * kj[e]
                sc.append(s / math.sqrt(hd))
            m = max(sc)
            ex = [math.exp(s - m) for s in sc]
            z = sum(ex)
            for e in range(hd):
                acc = 0.0
                for j in range(len(keys)):
                    acc += ex[j] / z * self.V[l][g][j][e]
                o.append(acc)
        return matvec(self.lw(l, "wo"), o)

    def mlp(self, l, x):
        c = self.c
        h = rms(x, self.lw(l, "mlp_norm"), c.rms_eps)
        gt = matvec(self.lw(l, "w_gate"), h)
        up = matvec(self.lw(l, "w_up"), h)
        act = [silu(gt[i]) * up[i] for i in range(len(gt))]
        return matvec(self.lw(l, "w_down"), act)

    def token(self, tok, pos):
        c = self.c
        x = list(self.w["embed"][tok])
        pend = {}
        for l in range(c.n_layers):
            if c.sequential:
                a = self.attn(l, x, pos)
                x = [x[i] + a[i] for i in range(len(x))]
                m = self.mlp(l, x)
                x = [x[i] + m[i] for i in range(len(x))]
            else:
                a = self.attn(l, x, pos)
                m = self.mlp(l, x)
                pend[l] = [a[i] + m[i] for i in range(len(x))]
                if l - c.lane_delay >= 0:
                    p = pend.pop(l - c.lane_delay)
                    x = [x[i] + p[i] for i in range(len(x))]
        for j in sorted(pend):
            x = [x[i] + pend[j][i] for i in range(len(x))]
        return matvec(self.w["lm_head"], rms(x, self.w["final_norm"], c.rms_eps))
