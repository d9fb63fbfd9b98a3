"""Host-side checks of the C ABI (no GPU needed, no kernel is launched):

* the library loads and exports every function include/spec_verify.h declares, and the
  binding's ctypes table covers exactly those;
* workspace queries are positive and grow with the problem;
* argument errors return the documented status before anything is enqueued, with a message;
* the product path never imports the oracle.
"""
import ctypes
import os
import re

import pytest

from speculative_decoding_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3
FAKE = 0x10000      # an aligned, never dereferenced address (validation fails before use)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from speculative_decoding_decode_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(spec_[a-z_0-9]+)\s*\(", text, flags=re.M)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)
    assert lib.spec_version() >> 16 == 1
    assert lib.spec_last_error() is not None


def test_workspace_queries(lib):
    a = lib.spec_verify_attn_workspace(1, 3, 8, 2, 256, 16, 512, 1024)
    b = lib.spec_verify_attn_workspace(8, 3, 8, 2, 256, 16, 512, 1024)
    g = lib.spec_verify_attn_workspace(1, 3, 8, 2, 256, 16, 512, 0)
    assert 0 < a <= b and a <= g
    l1 = lib.spec_lm_head_workspace(3, 2560, 262144)
    l2 = lib.spec_lm_head_workspace(96, 5376, 262144)
    assert 0 < l1 < l2
    c1 = lib.spec_accept_workspace(1, 2, 262144)
    c2 = lib.spec_accept_workspace(32, 2, 262144)
    assert 0 < c1 < c2
    assert lib.spec_lm_head_workspace(0, 8, 8) == 0
    assert b"positive" in lib.spec_last_error()
    assert lib.spec_verify_attn_workspace(1, 3, 8, 2, 96, 16, 512, 0) == 0
    assert b"head dim" in lib.spec_last_error()


def attn_call(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, ctx=FAKE, out=FAKE, B=1, K1=3, Hq=8, Hkv=2,
                D=256, ps=16, P=100, maxp=64, window=0, scale=0.0625, dtype=1, ws=FAKE,
                wsb=1 << 30)
    args.update(kw)
    return lib.spec_verify_attn(*args.values(), None)


def test_attn_argument_errors(lib):
    assert attn_call(lib, q=None) == EINVAL
    assert attn_call(lib, Hq=7) == EINVAL
    assert attn_call(lib, window=-1) == EINVAL
    assert attn_call(lib, D=96) == EUNSUP
    assert attn_call(lib, ps=32) == EUNSUP
    assert attn_call(lib, K1=65) == EUNSUP
    assert attn_call(lib, dtype=7) == EUNSUP
    assert attn_call(lib, q=FAKE + 4) == EINVAL
    assert b"alignment" in lib.spec_last_error()
    assert attn_call(lib, wsb=16) == EWS
    assert b"workspace" in lib.spec_last_error()
    assert attn_call(lib, B=1 << 25, K1=8, Hq=16, Hkv=4) == EUNSUP   # 2^32 output rows
    assert b"grid" in lib.spec_last_error()


def test_lm_head_argument_errors(lib):
    def call(**kw):
        a = dict(x=FAKE, w=FAKE, t=FAKE, logits=None, p=FAKE, R=3, H=2560, V=262144, dtype=1,
                 ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.spec_lm_head(*a.values(), None)

    assert call(p=None) == EINVAL
    assert call(R=0) == EINVAL
    assert call(H=2564) == EUNSUP
    assert call(dtype=3) == EUNSUP
    assert call(logits=FAKE + 8) == EINVAL
    assert call(wsb=8) == EWS
    assert call(ws=None) == EWS
    assert call(R=65536) == EUNSUP
    assert b"65535" in lib.spec_last_error()


def test_lm_head_noalloc_argument_errors(lib):
    # every rejection happens on the host, before the static array's address is looked up
    def call(**kw):
        a = dict(x=FAKE, w=FAKE, t=FAKE, logits=None, p=FAKE, R=3, H=2560, V=262144, dtype=1)
        a.update(kw)
        return lib.spec_lm_head_noalloc(*a.values(), None)

    assert call(p=None) == EINVAL
    assert call(R=0) == EINVAL
    assert call(H=2564) == EUNSUP
    assert call(x=FAKE + 8) == EINVAL
    # R * ceil(V / 256) * 12 bytes beyond the static array: 700 rows at V = 262144
    need = lib.spec_lm_head_workspace(700, 2560, 262144)
    assert need > 8 << 20
    assert call(R=700) == EUNSUP
    assert b"static array" in lib.spec_last_error()
    assert lib.spec_lm_head_workspace(681, 2560, 262144) <= 8 << 20


def test_lm_head_accept_argument_errors(lib):
    def call(**kw):
        a = dict(x=FAKE, w=FAKE, t=FAKE, d=FAKE, q=FAKE, u=None, seed=0, off=0, uo=None,
                 n=FAKE, tok=FAKE, B=1, k=2, H=2560, V=262144, dtype=1, ws=FAKE, wsb=1 << 32)
        a.update(kw)
        return lib.spec_lm_head_accept(*a.values(), None)

    assert call(q=None) == EINVAL
    assert call(B=0) == EINVAL
    assert call(k=64) == EUNSUP
    assert call(H=2564) == EUNSUP
    assert call(x=FAKE + 8) == EINVAL
    assert call(B=30000, k=2) == EUNSUP          # 90000 rows
    assert call(wsb=1 << 20) == EWS
    need = lib.spec_lm_head_accept_workspace(1, 2, 2560, 262144)
    # the contraction's exp values [R, V] fp32 plus statistics, sums and counters
    assert need > 3 * 262144 * 4
    assert lib.spec_lm_head_accept_workspace(1, 64, 8, 8) == 0


def test_accept_argument_errors(lib):
    def call(**kw):
        a = dict(d=FAKE, q=FAKE, p=FAKE, u=FAKE, n=FAKE, tok=FAKE, B=1, k=2, V=100, ws=FAKE,
                 wsb=1 << 20)
        a.update(kw)
        return lib.spec_accept(*a.values(), None)

    assert call(B=0) == EINVAL
    assert call(k=64) == EUNSUP
    assert call(q=None) == EINVAL
    assert call(k=0, q=None, d=None, wsb=1) == EWS   # q may be NULL when k == 0
    assert call(wsb=1) == EWS
    assert call(B=65536) == EUNSUP
    assert b"65535" in lib.spec_last_error()


def test_kv_argument_errors(lib):
    def append(**kw):
        a = dict(kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, table=FAKE, ctx=FAKE, B=1, K1=3, Hkv=2,
                 D=256, ps=16, P=100, maxp=64, dtype=1)
        a.update(kw)
        return lib.spec_kv_append(*a.values(), None)

    assert append(kn=None) == EINVAL
    assert append(B=0) == EINVAL
    assert append(ps=32) == EUNSUP
    assert append(D=12) == EUNSUP
    assert append(kp=FAKE + 8) == EINVAL
    assert append(B=1 << 26, K1=8, Hkv=4) == EUNSUP
    assert b"grid" in lib.spec_last_error()
    assert lib.spec_kv_commit(None, FAKE, 1, 3, None) == EINVAL
    assert lib.spec_kv_commit(FAKE, FAKE, 0, 3, None) == EINVAL


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "speculative_decoding_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", src), f
