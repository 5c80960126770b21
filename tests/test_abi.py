"""The C-ABI library without a GPU: it loads, exports what include/ckks_ks.h declares,
derives the same chain and roots as the oracle, and rejects bad arguments before any launch."""
import ctypes

import pytest

from oracle.chain import chain_primes as oracle_chain, min_root
from rns_ckks_key_amd import _lib
from rns_ckks_key_amd._lib import PCTX, U32, lib
from rns_ckks_key_amd.api import CkksError, Context, chain_primes

EINVAL, ERANGE, EUNSUPPORTED = -1, -2, -5


def test_every_declared_symbol_is_exported():
    names = _lib.header_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("log_n,bits,count", [(12, 30, 6), (16, 32, 48), (15, 32, 20)])
def test_chain_matches_oracle(log_n, bits, count):
    assert chain_primes(log_n, bits, count) == oracle_chain(1 << log_n, bits, count)


@pytest.mark.parametrize("log_n,L,K,dnum,bits", [(12, 4, 2, 2, 30), (16, 36, 12, 3, 32)])
def test_host_context_roots_match_oracle(log_n, L, K, dnum, bits):
    ctx = Context.for_chain(log_n, L, K, dnum, bits, max_batch=0)
    assert ctx.n == 1 << log_n and ctx.alpha == -(-L // dnum) and ctx.workspace_bytes == 0
    qs = oracle_chain(1 << log_n, bits, L + K)
    assert ctx.primes == qs
    idx = range(L + K) if log_n == 12 else (0, 17, 35, 36, 47)
    for t in idx:
        assert ctx.roots[t] == min_root(qs[t], 1 << log_n)
    ctx.close()


def _create(log_n, num_q, num_p, dnum, primes, max_batch=0):
    h = PCTX()
    arr = (U32 * len(primes))(*primes) if primes is not None else None
    st = lib.ckks_ctx_create(ctypes.byref(h), log_n, num_q, num_p, dnum, arr, max_batch)
    if st == 0:
        lib.ckks_ctx_destroy(h)
    return st


def test_ctx_create_rejects_bad_parameters():
    qs = oracle_chain(1 << 12, 30, 6)
    assert _create(12, 4, 2, 2, qs) == 0
    assert _create(12, 4, 2, 2, None) == EINVAL
    assert _create(11, 4, 2, 2, oracle_chain(1 << 11, 30, 6)) == EUNSUPPORTED
    assert _create(17, 4, 2, 2, qs) == EUNSUPPORTED
    bad = list(qs)
    bad[2] = 8193  # = 1 mod 2N but 3 * 2731
    assert _create(12, 4, 2, 2, bad) == ERANGE
    bad = list(qs)
    bad[1] = qs[1] + 2  # not = 1 mod 2N
    assert _create(12, 4, 2, 2, bad) == ERANGE
    bad = list(qs)
    bad[5] = qs[0]  # repeated prime
    assert _create(12, 4, 2, 2, bad) == ERANGE
    assert _create(12, 4, 1, 2, qs[:5]) == ERANGE  # special modulus narrower than a digit
    assert _create(12, 4, 2, 0, qs) == ERANGE
    msg = lib.ckks_last_error().decode()
    assert "dnum" in msg


def test_host_context_validates_calls_before_any_launch():
    ctx = Context.for_chain(12, 4, 2, 2, 30, max_batch=0)
    h = ctx.handle
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call stops before launching
    far = ctypes.c_void_p(0x1000000)  # 16 MiB on: clear of every [.][4..6][4096] range at `fake`
    seed = bytes(32)

    def ks(ct=fake, level=4, kb=fake, sd=seed, ka=None, g=5, out=far, batch=1):
        return lib.ckks_keyswitch(h, ct, level, kb, sd, ka, g, out, batch, None)

    assert ks(level=0) == ERANGE
    assert ks(level=5) == ERANGE
    assert ks(g=4) == ERANGE
    assert ks(g=2 * 4096 + 1) == ERANGE
    assert ks(batch=0) == ERANGE
    assert ks(ct=None) == EINVAL
    assert ks(kb=None) == EINVAL
    assert ks(out=None) == EINVAL
    assert ks(sd=None, ka=None) == EINVAL
    assert ks() == EINVAL and "host-only" in lib.ckks_last_error().decode()
    # out may not overlap ct or either key half ([2][4][4096] and [2][6][4096] words)
    words = 2 * 4 * 4096
    assert ks(out=ctypes.c_void_p(0x1000 + 4 * (words - 1))) == EINVAL and "overlaps ct" in lib.ckks_last_error().decode()
    hi = ctypes.c_void_p(0x200000)
    assert ks(ct=hi, out=ctypes.c_void_p(0x200000 - 4 * (words - 1))) == EINVAL
    assert "overlaps ct" in lib.ckks_last_error().decode()
    assert ks(ct=far, kb=fake, out=ctypes.c_void_p(0x1000 + 4 * 8000)) == EINVAL
    assert "overlaps key_b" in lib.ckks_last_error().decode()
    assert ks(ct=far, kb=ctypes.c_void_p(0x2000000), ka=fake, out=ctypes.c_void_p(0x1000 + 4 * 8000)) == EINVAL
    assert "overlaps key_a" in lib.ckks_last_error().decode()
    assert ks(kb=ctypes.c_void_p(0x2000000), out=ctypes.c_void_p(0x1000 + 4 * words)) == EINVAL  # adjacent is fine
    assert "host-only" in lib.ckks_last_error().decode()
    assert lib.ckks_modup(h, fake, 4, ctypes.c_void_p(0x1000 + 4 * 4096), 1, None) == EINVAL
    assert "overlaps" in lib.ckks_last_error().decode()
    assert lib.ckks_modup(h, fake, 4, ctypes.c_void_p(0x1000 + 4 * 4 * 4096), 1, None) == EINVAL
    assert "host-only" in lib.ckks_last_error().decode()
    assert lib.ckks_moddown(h, fake, 4, ctypes.c_void_p(0x1000 + 4 * 5 * 4096), 1, None) == EINVAL
    assert "overlaps x" in lib.ckks_last_error().decode()
    assert lib.ckks_moddown(h, fake, 4, ctypes.c_void_p(0x1000 + 4 * 6 * 4096), 1, None) == EINVAL
    assert "host-only" in lib.ckks_last_error().decode()
    assert lib.ckks_ntt_fwd(h, fake, 5, 2, 1, None) == ERANGE  # limbs 5..6 beyond 6 primes
    assert lib.ckks_ntt_fwd(h, None, 0, 2, 1, None) == EINVAL
    assert lib.ckks_ntt_inv(h, fake, 0, 0, 1, None) == ERANGE
    assert lib.ckks_modup(h, fake, 5, fake, 1, None) == ERANGE
    assert lib.ckks_moddown(h, fake, 0, fake, 1, None) == ERANGE
    assert lib.ckks_modup(h, None, 4, fake, 1, None) == EINVAL
    kb = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    gal = (U32 * 2)(5, 6)
    assert lib.ckks_keyswitch_hoisted(h, fake, 4, 2, kb, seed * 2, None, gal, fake, None) == ERANGE
    gal = (U32 * 2)(5, 25)
    assert lib.ckks_keyswitch_hoisted(h, fake, 4, 0, kb, seed * 2, None, gal, fake, None) == ERANGE
    assert lib.ckks_keyswitch_hoisted(h, fake, 4, 2, kb, None, None, gal, far, None) == EINVAL
    assert lib.ckks_keyswitch_hoisted(h, fake, 4, 2, kb, seed * 2, None, gal, fake, None) == EINVAL
    assert "overlaps ct" in lib.ckks_last_error().decode()
    kb2 = (ctypes.c_void_p * 2)(0x2000000, 0x1000000 + 4 * 2 * 2 * 4 * 4096 - 4)  # key 1 meets out's last word
    assert lib.ckks_keyswitch_hoisted(h, fake, 4, 2, kb2, seed * 2, None, gal, far, None) == EINVAL
    assert "overlaps key_b" in lib.ckks_last_error().decode()
    assert lib.ckks_keyswitch_hoisted(h, fake, 4, 2, kb, seed * 2, None, gal, far, None) == EINVAL
    assert "host-only" in lib.ckks_last_error().decode()
    assert lib.ckks_expand_a(h, None, fake, None) == EINVAL
    assert lib.ckks_rescale(h, fake, 1, far, 1, None) == ERANGE  # nothing to drop at level 1
    assert lib.ckks_rescale(h, fake, 5, far, 1, None) == ERANGE
    assert lib.ckks_rescale(h, None, 4, far, 1, None) == EINVAL
    assert lib.ckks_rescale(h, fake, 4, fake, 1, None) == EINVAL and "overlaps" in lib.ckks_last_error().decode()
    assert lib.ckks_rescale(h, fake, 4, far, 1, None) == EINVAL and "host-only" in lib.ckks_last_error().decode()

    def mrr(x=fake, level=4, kb=fake, sd=seed, ka=None, out=far, batch=1):
        return lib.ckks_mul_relin_rescale(h, x, x, level, kb, sd, ka, out, batch, None)

    assert mrr(level=1) == ERANGE
    assert mrr(batch=0) == ERANGE
    assert mrr(x=None) == EINVAL
    assert mrr(sd=None) == EINVAL
    assert mrr() == EINVAL and "host-only" in lib.ckks_last_error().decode()
    keys = (_lib.RotKey * 2)()
    keys[0].key_b = keys[1].key_b = 0x1000
    keys[0].galois_elt, keys[1].galois_elt = 5, 25

    def lt(n1=2, n2=2, baby=keys, giant=keys, diags=fake, level=4):
        return lib.ckks_linear_transform_bsgs(h, fake, level, n1, n2, baby, giant, diags, far, None)

    assert lt(n1=0) == ERANGE
    assert lt(n1=17) == ERANGE
    assert lt(n2=9) == ERANGE
    assert lt(level=5) == ERANGE
    assert lt(diags=None) == EINVAL
    assert lt(baby=None) == EINVAL
    keys[1].galois_elt = 4
    assert lt(n1=3) == ERANGE  # baby key 1 has an even Galois element
    keys[1].galois_elt = 25
    assert lt() == EINVAL and "host-only" in lib.ckks_last_error().decode()
    span = 2 * 4 * 4096 * 4  # bytes of one [2][4][4096] ciphertext

    def multi(*pairs, level=4):  # (ct, out) addresses of each item
        arr = (_lib.KsItem * len(pairs))()
        for it, (ct, out) in zip(arr, pairs):
            it.ct, it.out, it.key_b, it.level, it.galois_elt = ct, out, 0x1000, level, 5
        return lib.ckks_keyswitch_multi(h, len(pairs), arr, None)

    assert lib.ckks_keyswitch_multi(h, 0, None, None) == 0  # an empty stream is a no-op
    assert lib.ckks_keyswitch_multi(h, 2, None, None) == EINVAL
    base = 0x10000000
    assert multi((base, base + span), level=5) == ERANGE
    assert multi((base, base + span), (base + 2 * span, base + span + span // 2)) == EINVAL  # outputs overlap
    assert "outputs" in lib.ckks_last_error().decode()
    assert multi((base, base + span), (base + span + 4, base + 3 * span)) == EINVAL  # ct 1 inside out 0
    assert "item 1" in lib.ckks_last_error().decode()
    assert multi((base + 3 * span - 4, base + span), (base, base + 2 * span)) == EINVAL  # ct 0 reaches out 1
    assert "item 0" in lib.ckks_last_error().decode()
    # touching ranges and shared inputs are fine: the call gets as far as the device check
    assert multi((base, base + span), (base, base + 2 * span), (base + 4 * span, base + 3 * span)) == EINVAL
    assert "host-only" in lib.ckks_last_error().decode()
    assert lib.ckks_ctx_set_regen_blocks(h, 63) == ERANGE
    assert lib.ckks_ctx_set_regen_blocks(h, 64) == 0
    with pytest.raises(CkksError) as ei:
        _lib.check(ks(level=9))
    assert ei.value.name == "CKKS_ERANGE"
    ctx.close()


def test_conv_mfma_switch_validates_the_shape():
    # the matrix-core conversion exists for N = 2^16 with 9..12 primes per digit and special part
    tiny = Context.for_chain(12, 4, 2, 2, 30, max_batch=0)
    assert lib.ckks_ctx_set_conv_mfma(tiny.handle, 1) == EUNSUPPORTED
    assert lib.ckks_ctx_set_conv_mfma(tiny.handle, 0) == 0
    tiny.close()
    boot = Context.for_chain(16, 36, 12, 3, 32, max_batch=0)
    assert lib.ckks_ctx_set_conv_mfma(boot.handle, 1) == EINVAL  # host-only: no device tables
    assert "host-only" in lib.ckks_last_error().decode()
    boot.close()
    wide = Context.for_chain(16, 36, 6, 6, 32, max_batch=0)  # six primes per digit
    assert lib.ckks_ctx_set_conv_mfma(wide.handle, 1) == EUNSUPPORTED
    wide.close()
    assert lib.ckks_ctx_set_conv_mfma(None, 1) == EINVAL


def test_fusion_switch_needs_a_device_context():
    host = Context.for_chain(12, 4, 2, 2, 30, max_batch=0)
    assert lib.ckks_ctx_set_fused(host.handle, 0) == EINVAL  # host-only: there is no call to reroute
    assert "host-only" in lib.ckks_last_error().decode()
    host.close()
    assert lib.ckks_ctx_set_fused(None, 1) == EINVAL


def test_noalloc_keyswitch_validates_before_any_launch():
    # ckks_keyswitch_noalloc: the key-switch's checks, then its batch against the static
    # scratch array (96 MiB per GPU), not against max_batch
    boot = Context.for_chain(16, 36, 12, 3, 32, max_batch=0)
    h = boot.handle
    ct = ctypes.c_void_p(0x10000000)
    out = ctypes.c_void_p(0x40000000)
    kb = ctypes.c_void_p(0x70000000)
    seed = bytes(32)

    def nk(level=36, batch=1, ct=ct, out=out, g=5, sd=seed):
        return lib.ckks_keyswitch_noalloc(h, ct, level, kb, sd, None, g, out, batch, None)

    assert nk(batch=2) == ERANGE and "maximum" in lib.ckks_last_error().decode()  # 2 x 69 MiB
    assert nk(level=4, batch=4) == EINVAL and "host-only" in lib.ckks_last_error().decode()  # 4 x 21 MiB fits
    assert nk(level=4, batch=5) == ERANGE
    assert nk(batch=0) == ERANGE
    assert nk(level=37) == ERANGE
    assert nk(g=10) == ERANGE
    assert nk(sd=None) == EINVAL
    assert nk(out=ct) == EINVAL and "overlaps ct" in lib.ckks_last_error().decode()
    assert nk() == EINVAL and "host-only" in lib.ckks_last_error().decode()
    boot.close()


def test_library_is_built_from_the_sources_beside_it(monkeypatch, tmp_path):
    from rns_ckks_key_amd import build

    assert lib.ckks_build_id().decode() == build.source_digest()
    # the digest follows the content of every source and header
    copies = []
    for path in [build.os.path.join(build.CSRC, s) for s in build.SOURCES] + build.HEADERS:
        c = tmp_path / build.os.path.basename(path)
        c.write_bytes(open(path, "rb").read())
        copies.append(c)
    monkeypatch.setattr(build, "CSRC", str(tmp_path))
    monkeypatch.setattr(build, "HEADERS", [str(c) for c in copies[len(build.SOURCES):]])
    same = build.source_digest()
    assert same == lib.ckks_build_id().decode()
    copies[0].write_bytes(copies[0].read_bytes() + b"\n")
    assert build.source_digest() != same
    # a library built from other sources is refused at import
    with pytest.raises(ImportError, match="rebuild"):
        _lib._check_build()
