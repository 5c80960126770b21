"""Thin Python layer over the C-ABI: the same calls, on torch tensors.

Torch provides device memory and the current stream; the binding checks shapes,
passes `data_ptr()` and the stream handle, and raises CkksError on a non-zero
status.  Residue tensors are int32 or uint32 (bit patterns of uint32 residues),
contiguous, on the current CUDA (HIP) device.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import KERNEL_CLASSES, PCTX, U32, U64, CkksError, KsItem, RotKey, check, lib

__all__ = ["Context", "CkksError", "chain_primes", "to_device", "to_numpy"]


def chain_primes(log_n: int, bits: int, count: int) -> list[int]:
    buf = (U32 * count)()
    check(lib.ckks_chain_primes(log_n, bits, count, buf))
    return list(buf)


def to_device(a: np.ndarray, device: str | torch.device = "cuda") -> torch.Tensor:
    """uint32 numpy array -> int32 tensor holding the same bits, on `device`."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint64).astype(np.uint32))
    return torch.from_numpy(a.view(np.int32)).to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """int32/uint32 tensor -> uint32 numpy array."""
    x = t.detach().to("cpu").contiguous()
    if x.dtype == torch.int32:
        return x.numpy().view(np.uint32)
    return x.view(torch.int32).numpy().view(np.uint32)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None, shape: tuple[int, ...] | None, what: str) -> int | None:
    if t is None:
        return None
    if t.dtype not in (torch.int32, torch.uint32):
        raise TypeError(f"{what}: dtype {t.dtype}, want int32/uint32")
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor is not on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor is not contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, want {tuple(shape)}")
    return t.data_ptr()


def _seed(seed: bytes | None) -> bytes | None:
    if seed is None:
        return None
    if len(seed) != 32:
        raise ValueError("key seed must be 32 bytes")
    return bytes(seed)


class Context:
    """A prime chain, its constant tables and a workspace for `max_batch` ciphertexts (0: host only)."""

    def __init__(self, log_n: int, num_q: int, num_p: int, dnum: int, primes: list[int], max_batch: int):
        arr = (U32 * len(primes))(*primes)
        h = PCTX()
        check(lib.ckks_ctx_create(ctypes.byref(h), log_n, num_q, num_p, dnum, arr, max_batch))
        self._h = h
        n, L, K, d, alpha, mb = (U32() for _ in range(6))
        ws = U64()
        roots = (U32 * (num_q + num_p))()
        check(lib.ckks_ctx_info(h, ctypes.byref(n), ctypes.byref(L), ctypes.byref(K), ctypes.byref(d),
                                ctypes.byref(alpha), ctypes.byref(mb), ctypes.byref(ws), roots))
        self.log_n, self.n, self.L, self.K, self.dnum = log_n, n.value, L.value, K.value, d.value
        self.alpha, self.max_batch, self.workspace_bytes = alpha.value, mb.value, ws.value
        self.primes = list(primes)
        self.roots = list(roots)

    @classmethod
    def for_chain(cls, log_n: int, L: int, K: int, dnum: int, bits: int, max_batch: int) -> "Context":
        return cls(log_n, L, K, dnum, chain_primes(log_n, bits, L + K), max_batch)

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib.ckks_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def handle(self):
        return self._h

    def digits(self, level: int) -> int:
        return -(-level // self.alpha)

    def set_regen_blocks(self, blocks: int) -> None:
        check(lib.ckks_ctx_set_regen_blocks(self._h, blocks))

    def set_conv_mfma(self, on: bool) -> None:
        """Base conversions on the matrix cores (True) or the vector unit (False)."""
        check(lib.ckks_ctx_set_conv_mfma(self._h, 1 if on else 0))

    def set_fused(self, fused: bool) -> None:
        """keyswitch() with the inner product fused into ModDown (True, the default) or as separate launches."""
        check(lib.ckks_ctx_set_fused(self._h, 1 if fused else 0))

    def profile(self, enable: bool) -> None:
        """Bracket every launch with HIP events on its stream (measurement aid)."""
        check(lib.ckks_profile_enable(self._h, 1 if enable else 0))

    def profile_read(self) -> dict:
        """{kernel class: (summed ms, launches)} for the launches timed since profiling was enabled."""
        n = len(KERNEL_CLASSES)
        ms = (ctypes.c_double * n)()
        cnt = (U32 * n)()
        check(lib.ckks_profile_read(self._h, ms, cnt, n))
        return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}

    # ---- transforms
    def ntt_fwd(self, data: torch.Tensor, first_prime: int = 0) -> torch.Tensor:
        b, nl, n = data.shape
        check(lib.ckks_ntt_fwd(self._h, _ptr(data, (b, nl, self.n), "data"), first_prime, nl, b, _stream()))
        return data

    def ntt_inv(self, data: torch.Tensor, first_prime: int = 0) -> torch.Tensor:
        b, nl, n = data.shape
        check(lib.ckks_ntt_inv(self._h, _ptr(data, (b, nl, self.n), "data"), first_prime, nl, b, _stream()))
        return data

    # ---- key-switching steps
    def modup(self, c1: torch.Tensor, level: int, out: torch.Tensor | None = None) -> torch.Tensor:
        b = c1.shape[0]
        if out is None:
            out = torch.empty((b, self.digits(level), level + self.K, self.n), dtype=torch.int32, device=c1.device)
        check(lib.ckks_modup(self._h, _ptr(c1, (b, level, self.n), "c1"), level,
                             _ptr(out, (b, self.digits(level), level + self.K, self.n), "digits"), b, _stream()))
        return out

    def moddown(self, x: torch.Tensor, level: int, out: torch.Tensor | None = None) -> torch.Tensor:
        b = x.shape[0]
        if out is None:
            out = torch.empty((b, level, self.n), dtype=torch.int32, device=x.device)
        check(lib.ckks_moddown(self._h, _ptr(x, (b, level + self.K, self.n), "x"), level,
                               _ptr(out, (b, level, self.n), "out"), b, _stream()))
        return out

    def keyswitch(self, ct: torch.Tensor, level: int, key_b: torch.Tensor, galois: int = 1,
                  key_seed: bytes | None = None, key_a: torch.Tensor | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
        b = ct.shape[0]
        kshape = (self.dnum, self.L + self.K, self.n)
        if out is None:
            out = torch.empty((b, 2, level, self.n), dtype=torch.int32, device=ct.device)
        check(lib.ckks_keyswitch(self._h, _ptr(ct, (b, 2, level, self.n), "ct"), level, _ptr(key_b, kshape, "key_b"),
                                 _seed(key_seed), _ptr(key_a, kshape, "key_a"), galois,
                                 _ptr(out, (b, 2, level, self.n), "out"), b, _stream()))
        return out

    def keyswitch_noalloc(self, ct: torch.Tensor, level: int, key_b: torch.Tensor, galois: int = 1,
                          key_seed: bytes | None = None, key_a: torch.Tensor | None = None,
                          out: torch.Tensor | None = None) -> torch.Tensor:
        """keyswitch() with the library's static scratch array as workspace (the call allocates nothing)."""
        b = ct.shape[0]
        kshape = (self.dnum, self.L + self.K, self.n)
        if out is None:
            out = torch.empty((b, 2, level, self.n), dtype=torch.int32, device=ct.device)
        check(lib.ckks_keyswitch_noalloc(self._h, _ptr(ct, (b, 2, level, self.n), "ct"), level,
                                         _ptr(key_b, kshape, "key_b"), _seed(key_seed), _ptr(key_a, kshape, "key_a"),
                                         galois, _ptr(out, (b, 2, level, self.n), "out"), b, _stream()))
        return out

    def keyswitch_hoisted(self, ct: torch.Tensor, level: int, keys: list, out: torch.Tensor | None = None):
        """keys: list of (key_b, galois, key_seed or None, key_a or None)."""
        nk = len(keys)
        kshape = (self.dnum, self.L + self.K, self.n)
        if out is None:
            out = torch.empty((nk, 2, level, self.n), dtype=torch.int32, device=ct.device)
        kb = (ctypes.c_void_p * nk)(*[_ptr(k[0], kshape, "key_b") for k in keys])
        ka_list = [_ptr(k[3], kshape, "key_a") if k[3] is not None else None for k in keys]
        ka = (ctypes.c_void_p * nk)(*ka_list) if any(p is not None for p in ka_list) else None
        seeds = b"".join(_seed(k[2]) if k[2] is not None else bytes(32) for k in keys)
        gal = (U32 * nk)(*[k[1] for k in keys])
        check(lib.ckks_keyswitch_hoisted(self._h, _ptr(ct, (2, level, self.n), "ct"), level, nk, kb, seeds, ka,
                                         gal, _ptr(out, (nk, 2, level, self.n), "out"), _stream()))
        return out

    def keyswitch_multi(self, items: list) -> list:
        """items: list of (ct [2][l][N], level, key_b, galois, key_seed or None, key_a or None, out or None).

        One key-switch per item, bit-identical to separate keyswitch calls; returns the outputs."""
        kshape = (self.dnum, self.L + self.K, self.n)
        arr = (KsItem * len(items))()
        outs = []
        for i, (ct, level, key_b, galois, seed, key_a, out) in enumerate(items):
            if out is None:
                out = torch.empty((2, level, self.n), dtype=torch.int32, device=ct.device)
            outs.append(out)
            it = arr[i]
            it.ct = _ptr(ct, (2, level, self.n), "ct")
            it.out = _ptr(out, (2, level, self.n), "out")
            it.key_b = _ptr(key_b, kshape, "key_b")
            it.key_a = _ptr(key_a, kshape, "key_a") if key_a is not None else None
            if key_a is None:
                ctypes.memmove(it.key_seed, _seed(seed), 32)
            it.level = level
            it.galois_elt = galois
        check(lib.ckks_keyswitch_multi(self._h, len(items), arr, _stream()))
        return outs

    def rescale(self, ct: torch.Tensor, level: int, out: torch.Tensor | None = None) -> torch.Tensor:
        """[batch][2][level][N] -> [batch][2][level-1][N]: drop the last active prime (floor convention)."""
        b = ct.shape[0]
        if out is None:
            out = torch.empty((b, 2, level - 1, self.n), dtype=torch.int32, device=ct.device)
        check(lib.ckks_rescale(self._h, _ptr(ct, (b, 2, level, self.n), "ct"), level,
                               _ptr(out, (b, 2, level - 1, self.n), "out"), b, _stream()))
        return out

    def mul_relin_rescale(self, x: torch.Tensor, y: torch.Tensor, level: int, key_b: torch.Tensor,
                          key_seed: bytes | None = None, key_a: torch.Tensor | None = None,
                          out: torch.Tensor | None = None) -> torch.Tensor:
        """Rescale(Relinearise(x (x) y)) with the s^2 -> s key: [batch][2][level-1][N]."""
        b = x.shape[0]
        kshape = (self.dnum, self.L + self.K, self.n)
        if out is None:
            out = torch.empty((b, 2, level - 1, self.n), dtype=torch.int32, device=x.device)
        check(lib.ckks_mul_relin_rescale(self._h, _ptr(x, (b, 2, level, self.n), "x"),
                                         _ptr(y, (b, 2, level, self.n), "y"), level, _ptr(key_b, kshape, "key_b"),
                                         _seed(key_seed), _ptr(key_a, kshape, "key_a"),
                                         _ptr(out, (b, 2, level - 1, self.n), "out"), b, _stream()))
        return out

    def _rot_keys(self, keys: list):
        kshape = (self.dnum, self.L + self.K, self.n)
        arr = (RotKey * max(1, len(keys)))()
        for i, (key_b, galois, seed, key_a) in enumerate(keys):
            arr[i].key_b = _ptr(key_b, kshape, "key_b")
            arr[i].key_a = _ptr(key_a, kshape, "key_a") if key_a is not None else None
            if key_a is None:
                ctypes.memmove(arr[i].key_seed, _seed(seed), 32)
            arr[i].galois_elt = galois
        return arr

    def linear_transform_bsgs(self, ct: torch.Tensor, level: int, diags: torch.Tensor, baby: list, giant: list,
                              out: torch.Tensor | None = None) -> torch.Tensor:
        """sum_j Rot_j(ModDown(sum_k D[j][k] * R_k)); baby/giant: lists of (key_b, galois, seed or None, key_a or None).

        diags: [n2][n1][level+K][N]; len(baby) = n1 - 1, len(giant) = n2 - 1."""
        n2, n1 = diags.shape[0], diags.shape[1]
        if out is None:
            out = torch.empty((2, level, self.n), dtype=torch.int32, device=ct.device)
        check(lib.ckks_linear_transform_bsgs(self._h, _ptr(ct, (2, level, self.n), "ct"), level, n1, n2,
                                             self._rot_keys(baby), self._rot_keys(giant),
                                             _ptr(diags, (n2, n1, level + self.K, self.n), "diags"),
                                             _ptr(out, (2, level, self.n), "out"), _stream()))
        return out

    def expand_a(self, seed: bytes, out: torch.Tensor | None = None, device="cuda") -> torch.Tensor:
        kshape = (self.dnum, self.L + self.K, self.n)
        if out is None:
            out = torch.empty(kshape, dtype=torch.int32, device=device)
        check(lib.ckks_expand_a(self._h, _seed(seed), _ptr(out, kshape, "key_a"), _stream()))
        return out
