"""One-hot gather probes: inputs whose exact attention output names the cache slot it came from.

Construction (no attention arithmetic: every expected value follows from the
construction alone, and the oracle reproduces it exactly on the small cases):

* V.  The token in physical block p, kv head g, slot s holds at element d a
  small integer in 0..15 (exact in fp32, bf16 and E4M3): for d % 8 = 0..3 the
  four base-16 digits of p, 4: g, 5 and 6: the two base-16 digits of s, 7:
  d // 8.  A wrong block, head, slot or element shows as a wrong integer.
* q.  Query i of row b, query head h = g*G + j, is the unit vector e_c of its
  column c = (i*G + j) mod 128 (shared-prefix rows: columns by the row's rank
  among the probed rows, so rows that can see the same blocks use different
  columns).
* K.  Zero, except K[p*][g][s*][c] = BIG at each column's target slot.  The
  target of column c is a token every query of that column may see (causal
  rows: at or before the earliest such query's position).  The query's score
  is then BIG*scale (about 1,448 at scale 1/sqrt(128)) on the target and 0 on
  every other token; exp(-1448) is 0 in fp32 and fp64, so the output is the
  target's V exactly: digits(p*, g, s*) * v_scale[g].
* FP8 pools: BIG is the code 0x7E (448) with k_scale[g] = 2^(6 + g % 2); the V
  scales are powers of two, 2^-(g % 3), so the expected values stay exact.

Targets sweep, over the launches r = 0, 1, ..., the first and last slot of
every block of the row, its last token and its new tokens (the causal
diagonal), rotating over the columns so that a few launches cover them all.

The block-table indexing this pins is the ordered per-request block list of
"How does TensorRT-LLM work" (outcomeschool.com), section "The paged KV
cache", over non-contiguous blocks ("Introduction to TensorRT-LLM",
dileepadev.github.io, section "2. Paged KV Cache").
"""
from __future__ import annotations

import numpy as np

import pa_inputs

BIG = 16384.0
BIG_BF16 = np.uint16(0x4680)          # 16384.0
ONE_BF16 = np.uint16(0x3F80)          # 1.0
FP8_BIG_CODE = np.uint8(0x7E)         # E4M3 448.0
NAN = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}


def fp8_k_scale(hkv):
    return np.array([2.0 ** (6 + g % 2) for g in range(hkv)], np.float32)


def fp8_v_scale(hkv):
    return np.array([2.0 ** -(g % 3) for g in range(hkv)], np.float32)


def digit_lut(fmt):
    """Stored encodings of the integers 0..15 in ``fmt``."""
    import torch
    x = torch.arange(16, dtype=torch.float32)
    if fmt == "f32":
        return x.numpy()
    if fmt == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if fmt == "fp8":
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(fmt)


def slot_digits(p, g, s):
    """[..., 128] float64 integer vector held by the token at (block p, kv head g, slot s)."""
    p, g, s = np.broadcast_arrays(np.asarray(p, np.int64), np.asarray(g, np.int64), np.asarray(s, np.int64))
    seven = np.stack([p & 15, (p >> 4) & 15, (p >> 8) & 15, (p >> 12) & 15, g & 15, s & 15, (s >> 4) & 15], -1)
    out = np.empty(p.shape + (16, 8), np.float64)
    out[..., :7] = seven[..., None, :]
    out[..., 7] = np.arange(16)
    return out.reshape(p.shape + (128,))


def digit_pool(num_blocks, hkv, bs, fmt):
    """V pool [num_blocks][hkv][bs][128] in storage format ``fmt`` holding slot_digits."""
    assert num_blocks <= 1 << 16 and bs <= 256 and hkv <= 16
    lut = digit_lut(fmt)
    p = np.arange(num_blocks)[:, None, None]
    g = np.arange(hkv)[None, :, None]
    s = np.arange(bs)[None, None, :]
    p, g, s = np.broadcast_arrays(p, g, s)
    seven = np.stack([p & 15, (p >> 4) & 15, (p >> 8) & 15, (p >> 12) & 15, g & 15, s & 15, (s >> 4) & 15], -1)
    out = np.empty((num_blocks, hkv, bs, 16, 8), lut.dtype)
    out[..., :7] = lut[seven][..., None, :]
    out[..., 7] = lut[np.arange(16)]
    return out.reshape(num_blocks, hkv, bs, 128)


def _candidates(L, n, bs):
    """First and last slot of every block, the last token and the new tokens (the diagonal)."""
    nb = (L + bs - 1) // bs
    j = np.arange(nb)
    c = np.concatenate([j * bs, np.minimum(j * bs + bs - 1, L - 1), [L - 1], np.arange(L - n, L)])
    return np.unique(c)


class OneHotProbe:
    """Targets, queries and expected outputs of one-hot probes on workload ``w``.

    ``prepare()`` replaces w's V pool (and FP8 scales) with the digit encoding;
    ``launch(r)`` gives launch r's queries, K entries and expected outputs.
    """

    def __init__(self, w, shared_rows=False):
        self.w = w
        self.Hq, self.Hkv, self.D = w.num_q_heads, w.num_kv_heads, w.head_dim
        assert self.D == 128
        self.G = self.Hq // self.Hkv
        self.bs = w.block_size
        self.shared_rows = shared_rows
        self.qsl = w.q_start_loc
        self.cands = [_candidates(int(w.seq_lens[b]), int(w.q_lens[b]), self.bs) for b in range(w.num_seqs)]
        if w.kv_fmt == "fp8":
            self.k_scale, self.v_scale = fp8_k_scale(self.Hkv), fp8_v_scale(self.Hkv)
        else:
            self.k_scale = self.v_scale = None

    # ---------------------------------------------------------------- inputs
    def prepare(self, poison=True):
        """Digit-encoded V pool and the FP8 scales, on the host workload."""
        w = self.w
        w.v_pool = digit_pool(w.num_blocks, self.Hkv, self.bs, w.kv_fmt)
        if w.kv_fmt == "fp8":
            w.k_scale, w.v_scale = self.k_scale.copy(), self.v_scale.copy()
        w.k_pool = np.zeros_like(w.k_pool)
        if poison:
            pa_inputs.poison_pool(w)

    def num_launches(self):
        """Launches for every candidate of every row to be some column's target at least once."""
        per = []
        for b in range(self.w.num_seqs):
            n = int(self.w.q_lens[b])
            cols = min(128, n * self.G) if not self.shared_rows else self.G
            per.append(-(-len(self.cands[b]) // (cols * self.Hkv)))
        return max(per) if per else 1

    def active_rows(self, r):
        """Rows probed in launch r (shared-prefix rows take distinct columns, 128 // G per launch)."""
        B = self.w.num_seqs
        if not self.shared_rows:
            return np.arange(B)
        per = 128 // self.G
        k = -(-B // per)
        part = r % k
        return np.arange(part * per, min(B, (part + 1) * per))

    def launch(self, r):
        """Launch r: (q storage [total_q][Hq][D], K entries (phys, g, slot, col) as int arrays,
        expected float64 [total_q][Hq][D], bool [total_q] of the query rows whose output is exact)."""
        w, G, Hkv = self.w, self.G, self.Hkv
        qf = np.zeros((w.total_q, self.Hq, self.D), np.float32)
        exp = np.zeros((w.total_q, self.Hq, self.D), np.float64)
        checked = np.zeros(w.total_q, bool)
        ents = []
        for rank, b in enumerate(self.active_rows(r)):
            L, n, q0 = int(w.seq_lens[b]), int(w.q_lens[b]), int(self.qsl[b])
            cand = self.cands[b]
            checked[q0:q0 + n] = True
            for g in range(Hkv):
                for j in range(G):
                    if self.shared_rows:
                        assert n == 1
                        cols = {rank * G + j: [0]}
                    else:
                        cols = {}
                        for i in range(n):
                            cols.setdefault((i * G + j) % 128, []).append(i)
                    for c, qs in cols.items():
                        vis = L - n + min(qs)
                        cc = cand[cand <= vis]
                        k = (r * Hkv * 128 + g * 128 + c + 7 * b) % len(cc)
                        t = int(cc[k])
                        p, s = int(w.block_table[b, t // self.bs]), t % self.bs
                        ents.append((p, g, s, c))
                        val = slot_digits(p, g, s)
                        if self.v_scale is not None:
                            val = val * float(self.v_scale[g])
                        for i in qs:
                            qf[q0 + i, g * G + j, c] = 1.0
                            exp[q0 + i, g * G + j] = val
        ents = np.array(sorted(set(ents)), np.int64).reshape(-1, 4)
        q = qf if w.q_fmt == "f32" else pa_inputs.to_bf16_bits(qf)
        return q, ents, exp, checked

    def big_code(self):
        return {"f32": np.float32(BIG), "bf16": BIG_BF16, "fp8": FP8_BIG_CODE}[self.w.kv_fmt]

    def apply_host(self, r, poison=True):
        """Launch r's q and K written into the host workload; returns (expected, checked)."""
        w = self.w
        q, ents, exp, checked = self.launch(r)
        w.q = q
        w.k_pool[...] = 0
        w.k_pool[ents[:, 0], ents[:, 1], ents[:, 2], ents[:, 3]] = self.big_code()
        if poison:
            pa_inputs.poison_pool(w)
        return exp, checked


class DeviceProbe:
    """The same probe with the pools on the GPU: K is cleared and re-targeted in place."""

    def __init__(self, probe, dev):
        import torch
        self.p, self.d = probe, dev
        w = probe.w
        mask = pa_inputs.poison_mask(w)                       # [nb, bs]
        self.poison = torch.from_numpy(mask).cuda() if mask.any() else None
        self.k_raw = self._raw(dev["k_pool"])
        self.v_raw = self._raw(dev["v_pool"])
        nan = NAN[w.kv_fmt]
        self.nan = torch.tensor(np.array([nan]).view({"f32": np.float32, "bf16": np.int16, "fp8": np.uint8}[w.kv_fmt]),
                                device="cuda")[0]
        self.big = torch.tensor(np.array([probe.big_code()]).view(
            {"f32": np.float32, "bf16": np.int16, "fp8": np.uint8}[w.kv_fmt]), device="cuda")[0]
        if self.poison is not None:
            self._poison(self.v_raw)

    @staticmethod
    def _raw(t):
        import torch
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t

    def _poison(self, raw):
        raw.permute(0, 2, 1, 3)[self.poison] = self.nan

    def set_launch(self, r):
        """Launch r's q and K on the device; returns (expected, checked)."""
        import torch
        q, ents, exp, checked = self.p.launch(r)
        self.k_raw.zero_()
        idx = torch.from_numpy(ents).cuda()
        self.k_raw[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]] = self.big
        if self.poison is not None:
            self._poison(self.k_raw)
        qd = self.d["q"]
        if qd.dtype == torch.bfloat16:
            qd.view(torch.int16).copy_(torch.from_numpy(q.view(np.int16)).cuda())
        else:
            qd.copy_(torch.from_numpy(q).cuda())
        torch.cuda.synchronize()
        return exp, checked
