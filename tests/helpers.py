"""Shared helpers for the GPU tests: run a stream through a ring and through
the oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import chunked_attention_amd as kv
from oracle import attention as O1
from oracle import fp8 as O3

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
# lse of bf16 rings is that of the weights applied: reference + ln of the sum
# of the bf16-rounded probabilities that O is divided by.  Each weight is
# rounded once to bf16 (8 significant bits, relative error <= 2^-8), so it is
# within ln(1 + 2^-8) of the exact log-sum-exp; the slack covers the float32
# arithmetic.
LSE_BF16_BOUND = float(np.log1p(2.0 ** -8)) + 5e-5
FP8_MAX_ABS = 6e-2


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


def compare(o_gpu: torch.Tensor, o_ref: np.ndarray, heads=None) -> dict:
    g = to_f64(o_gpu)
    r = o_ref
    if heads is not None:
        g = g[:, heads]
        r = r[:, heads] if r.shape[1] != len(heads) else r
    diff = g - r
    nref = np.linalg.norm(r)
    per_head = np.abs(diff).max(axis=(0, 2))
    return {
        "max_abs": float(np.abs(diff).max()),
        "rel_l2": float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff)),
        "worst_head": int(per_head.argmax()),
        "finite": bool(np.isfinite(g).all()),
    }


def assert_bf16_parity(stats: dict, what: str = "") -> None:
    assert stats["finite"], f"{what}: non-finite output"
    assert stats["max_abs"] <= BF16_MAX_ABS, f"{what}: {stats}"
    assert stats["rel_l2"] <= BF16_REL_L2, f"{what}: {stats}"


def fp8_roundtrip_tokens(x: torch.Tensor) -> np.ndarray:
    """float64 values an fp8 ring holds for token-major x [rows, H, d]."""
    return O3.roundtrip_segment(x.to(torch.float32).numpy())


class StreamRun:
    """Drives one ring and the oracle over a synthetic stream."""

    def __init__(self, stream, ring: kv.Ring, fp8: bool = False, heads=None):
        self.s = stream
        self.w = stream.w
        self.ring = ring
        self.fp8 = fp8
        self.heads = heads
        self.last_vmax = 0.0     # largest |v| of the current chunk's staged values
        ck, cv = stream.kv_cond() if self.w.cond_tokens else (None, None)
        rk, rv = stream.kv_ref() if self.w.ref_tokens else (None, None)
        self.oracle = O1.StreamOracle(self.w.window, self.w.scale,
                                      self._ref(ck), self._ref(cv), self._ref(rk),
                                      self._ref(rv))
        if ck is not None:
            ring.cond(ck.cuda(), cv.cuda())
        if rk is not None:
            ring.ref(rk.cuda(), rv.cuda())

    def _ref(self, x):
        # the sampled heads first: the fp8 scales are per (head, segment), so
        # the round trip of a head does not depend on the other heads
        if x is None:
            return None
        if self.heads is not None:
            x = x[:, self.heads]
        if self.fp8:
            return fp8_roundtrip_tokens(x)
        return O1.as_f64(x)

    def chunk(self, t: int, check: bool = True, lse: bool = False):
        """Stage + attend every step, commit, evict.  Returns per-step
        (gpu_out, ref_out, stats)."""
        results = []
        src = self.w.source_tokens > 0
        for step in range(self.w.steps):
            k, v = self.s.kv_noisy(t, step)
            q = self.s.q(t, step)
            sk = sv = None
            if src:
                sk, sv = self.s.kv_src(t, step)
                q = torch.cat([q, self.s.q_src(t, step)])
            if check:
                self.last_vmax = float(np.abs(self._ref(v)).max())
            if src:
                self.ring.stage(torch.cat([k, sk]).cuda(), torch.cat([v, sv]).cuda())
            else:
                self.ring.stage(k.cuda(), v.cuda())
            lse_t = torch.empty(self.w.heads, q.shape[0], dtype=torch.float32,
                                device="cuda") if lse else None
            o = self.ring.attention(q.cuda(), lse=lse_t)
            if check:
                qr = O1.as_f64(q)
                if self.heads is not None:
                    qr = qr[:, self.heads]
                ref, ref_lse = self.oracle.attend(t, qr, self._ref(k), self._ref(v),
                                                  src_k=self._ref(sk), src_v=self._ref(sv))
                stats = compare(o, ref, self.heads)
                if lse:
                    g = to_f64(lse_t)
                    if self.heads is not None:
                        g = g[self.heads]
                    stats["lse_max_abs"] = float(np.abs(g - ref_lse).max())
                results.append((o, ref, stats))
            else:
                results.append((o, None, None))
        kc, vc = self.s.kv_clean(t)
        if src:
            skc, svc = self.s.kv_src_clean(t)
            self.ring.commit(torch.cat([kc, skc]).cuda(), torch.cat([vc, svc]).cuda())
        else:
            self.ring.commit(kc.cuda(), vc.cuda())
        self.oracle.commit(t, self._ref(kc), self._ref(vc))
        self.ring.evict()
        return results
