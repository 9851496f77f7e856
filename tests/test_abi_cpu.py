"""The C-ABI library loads, exports every declared symbol and validates arguments.

CPU only: every call here fails host-side validation before any HIP call, so no
device is needed and no kernel is launched. The memra README's recent-fixes list
states the rule these tests follow: a truncated or malformed input yields a
contextual error, never a crash, for every byte-prefix of a valid buffer.
"""

import ctypes
import os
import re

import pytest

import gguf_block_quantized_qmv_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = q.lib

OK, NULL, SHAPE, SIZE, ALIGN, RANGE, WORKSPACE, ALIAS, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8

# Fake, never dereferenced device addresses (validation rejects every call below first).
A = 0x7F0000000000
W, X, Y, WS = A, A + (1 << 32), A + (2 << 32), A + (3 << 32)
V = ctypes.c_void_p


def _header_functions():
    with open(os.path.join(ROOT, "include", "qmv.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(qm[mv]_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_lists_the_expected_entry_points():
    assert _header_functions() == sorted([
        "qmv_version", "qmv_strerror", "qmv_last_error", "qmv_q8_0", "qmv_q4_k", "qmv_iq4_xs", "qmv_q4_k_moe_workspace",
        "qmv_q4_k_moe", "qmv_q4_k_moe_prefill",
        "qmv_q4_k_moe_prefill_workspace", "qmv_dequant_iq4_xs_f32", "qmv_iq4_xs_moe_workspace", "qmv_iq4_xs_moe",
        "qmv_q5_k", "qmv_dequant_q5_k_f32", "qmv_q6_k", "qmv_dequant_q6_k_f32", "qmv_q4_0",
        "qmv_dequant_q4_0_f32",
        "qmm_q4_k_prefill_workspace", "qmm_q4_k_prefill", "qmv_dequant_q4_k_f32", "qmv_dequant_q4_k_bf16",
        "qmv_dequant_q8_0_f32", "qmv_stream_read", "qmv_q4_k_moe_noalloc", "qmv_q4_k_pair"])


def test_library_exports_every_declared_symbol():
    for name in _header_functions():
        assert hasattr(L, name), name
    assert set(_header_functions()) == set(q.EXPORTS)


def test_version_and_strerror():
    assert L.qmv_version() > 0
    for code in (OK, NULL, SHAPE, SIZE, ALIGN, RANGE, WORKSPACE, ALIAS, HIP, -99, 7):
        s = L.qmv_strerror(code)
        assert isinstance(s, bytes) and len(s) > 1


def q4k(w=W, nbytes=None, x=X, y=Y, m=1, n=2, k=256):
    nbytes = q.q4_k_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_q4_k(V(w), nbytes, V(x), V(y), m, n, k, None)


def q80(w=W, nbytes=None, x=X, y=Y, m=1, n=2, k=64):
    nbytes = q.q8_0_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_q8_0(V(w), nbytes, V(x), V(y), m, n, k, None)


def test_q4_k_validation():
    assert q4k(w=0) == NULL and q4k(x=0) == NULL and q4k(y=0) == NULL
    assert q4k(m=0) == RANGE and q4k(m=5) == RANGE
    assert q4k(n=0) == SHAPE and q4k(k=0) == SHAPE and q4k(k=255) == SHAPE and q4k(k=384) == SHAPE
    assert q4k(w=W + 8) == ALIGN and q4k(x=X + 2) == ALIGN and q4k(y=Y + 2) == ALIGN
    assert q4k(m=4, k=19456) == RANGE                   # activations exceed the LDS stage
    assert q4k(y=W + 64) == ALIAS                        # output inside the weights
    assert q4k(y=X, x=X) == ALIAS


def test_q4_k_every_truncated_or_padded_size_is_an_error():
    n, k = 2, 512
    full = q.q4_k_bytes(n, k)
    for b in range(full):
        assert q4k(nbytes=b, n=n, k=k) == SIZE, b
    assert q4k(nbytes=full + 1, n=n, k=k) == SIZE
    assert q4k(nbytes=2 * full, n=n, k=k) == SIZE


W1 = W + (1 << 30)   # the second matrix of a pair
Y1 = Y + (1 << 30)


def q4kp(w0=W, w1=W1, nbytes=None, x=X, y0=Y, y1=Y1, m=1, n=2, k=256):
    nbytes = q.q4_k_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_q4_k_pair(V(w0), V(w1), nbytes, V(x), V(y0), V(y1), m, n, k, None)


def test_q4_k_pair_validation():
    assert q4kp(w0=0) == NULL and q4kp(w1=0) == NULL and q4kp(x=0) == NULL and q4kp(y0=0) == NULL
    assert q4kp(y1=0) == NULL
    assert q4kp(m=0) == RANGE and q4kp(m=5) == RANGE
    assert q4kp(n=0) == SHAPE and q4kp(k=0) == SHAPE and q4kp(k=255) == SHAPE and q4kp(k=384) == SHAPE
    assert q4kp(w0=W + 8) == ALIGN and q4kp(w1=W1 + 8) == ALIGN and q4kp(x=X + 2) == ALIGN
    assert q4kp(y0=Y + 2) == ALIGN and q4kp(y1=Y1 + 2) == ALIGN
    assert q4kp(m=4, k=19456) == RANGE                  # activations exceed the LDS stage
    assert q4kp(y0=W + 64) == ALIAS and q4kp(y1=W1 + 64) == ALIAS and q4kp(y1=W + 64) == ALIAS
    assert q4kp(y0=X, x=X) == ALIAS and q4kp(y1=X + 4, x=X) == ALIAS
    assert q4kp(y1=Y + 4) == ALIAS                      # the outputs overlap each other
    full = q.q4_k_bytes(2, 512)
    for b in (0, full - 1, full + 1, 2 * full):
        assert q4kp(nbytes=b, k=512) == SIZE, b
    # one grid covers 2n rows: each matrix may have at most half the row limit
    assert q4kp(n=(1 << 29) + 1, k=256, nbytes=q.q4_k_bytes((1 << 29) + 1, 256)) == RANGE


def q5k(w=W, nbytes=None, x=X, y=Y, m=1, n=2, k=256):
    nbytes = q.q5_k_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_q5_k(V(w), nbytes, V(x), V(y), m, n, k, None)


def test_q5_k_validation():
    assert q5k(w=0) == NULL and q5k(x=0) == NULL and q5k(y=0) == NULL
    assert q5k(m=0) == RANGE and q5k(m=5) == RANGE
    assert q5k(n=0) == SHAPE and q5k(k=0) == SHAPE and q5k(k=255) == SHAPE and q5k(k=384) == SHAPE
    assert q5k(w=W + 8) == ALIGN and q5k(x=X + 2) == ALIGN and q5k(y=Y + 2) == ALIGN
    assert q5k(m=4, k=19456) == RANGE
    assert q5k(y=W + 64) == ALIAS
    full = q.q5_k_bytes(2, 512)
    assert q.q5_k_bytes(2, 512) == 2 * 2 * 176
    for b in list(range(full)) + [full + 1, full + 176, q.q4_k_bytes(2, 512)]:
        assert q5k(nbytes=b, k=512) == SIZE, b
    nb = q.q5_k_bytes(2, 256)
    f = L.qmv_dequant_q5_k_f32
    assert f(V(0), nb, V(Y), 2, 256, None) == NULL and f(V(W), nb - 1, V(Y), 2, 256, None) == SIZE
    assert f(V(W), nb, V(Y + 4), 2, 256, None) == ALIGN and f(V(W), nb, V(W), 2, 256, None) == ALIAS


def q40(w=W, nbytes=None, x=X, y=Y, m=1, n=2, k=256):
    nbytes = q.q4_0_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_q4_0(V(w), nbytes, V(x), V(y), m, n, k, None)


def test_q4_0_validation():
    assert q40(w=0) == NULL and q40(x=0) == NULL and q40(y=0) == NULL
    assert q40(m=0) == RANGE and q40(m=5) == RANGE
    assert q40(n=0) == SHAPE and q40(k=0) == SHAPE and q40(k=32) == SHAPE and q40(k=224) == SHAPE
    assert q40(k=288) == SHAPE and q40(k=255) == SHAPE
    assert q40(w=W + 8) == ALIGN and q40(w=W + 2) == ALIGN and q40(x=X + 2) == ALIGN and q40(y=Y + 2) == ALIGN
    assert q40(m=4, k=19456) == RANGE
    assert q40(y=W + 64) == ALIAS
    full = q.q4_0_bytes(2, 512)
    assert full == 2 * 16 * 18
    # (a Q4_K matrix of the same shape has the same size: 144 bytes per 256 weights)
    for b in list(range(full)) + [full + 1, full + 18, q.q5_k_bytes(2, 512)]:
        assert q40(nbytes=b, k=512) == SIZE, b
    f = L.qmv_dequant_q4_0_f32
    nb = q.q4_0_bytes(2, 32)
    assert f(V(0), nb, V(Y), 2, 32, None) == NULL and f(V(W), nb - 1, V(Y), 2, 32, None) == SIZE
    assert f(V(W), nb, V(Y + 4), 2, 32, None) == ALIGN and f(V(W), nb, V(W), 2, 32, None) == ALIAS
    assert f(V(W + 1), nb, V(Y), 2, 32, None) == ALIGN and f(V(W), nb, V(Y), 2, 16, None) == SHAPE


def q6k(w=W, nbytes=None, x=X, y=Y, m=1, n=2, k=256):
    nbytes = q.q6_k_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_q6_k(V(w), nbytes, V(x), V(y), m, n, k, None)


def test_q6_k_validation():
    assert q6k(w=0) == NULL and q6k(x=0) == NULL and q6k(y=0) == NULL
    assert q6k(m=0) == RANGE and q6k(m=5) == RANGE
    assert q6k(n=0) == SHAPE and q6k(k=0) == SHAPE and q6k(k=255) == SHAPE and q6k(k=384) == SHAPE
    assert q6k(w=W + 8) == ALIGN and q6k(w=W + 2) == ALIGN and q6k(x=X + 2) == ALIGN and q6k(y=Y + 2) == ALIGN
    # the LDS stage: m * k * 2.25 bytes; m = 4 allows k up to 18176, m = 3 up to 24064
    assert q6k(m=4, k=18176, n=1, y=Y + 2) == ALIGN   # passes the LDS check, stops at alignment
    assert q6k(m=3, k=24064, n=1, y=Y + 2) == ALIGN
    assert q6k(m=4, k=18432, n=1) == RANGE and q6k(m=3, k=24320, n=1) == RANGE
    assert q6k(y=W + 64) == ALIAS
    full = q.q6_k_bytes(2, 512)
    assert full == 2 * 2 * 210
    for b in list(range(full)) + [full + 1, full + 210, q.q5_k_bytes(2, 512), q.q4_k_bytes(2, 512)]:
        assert q6k(nbytes=b, k=512) == SIZE, b
    nb = q.q6_k_bytes(2, 256)
    f = L.qmv_dequant_q6_k_f32
    assert f(V(0), nb, V(Y), 2, 256, None) == NULL and f(V(W), nb - 1, V(Y), 2, 256, None) == SIZE
    assert f(V(W), nb, V(Y + 4), 2, 256, None) == ALIGN and f(V(W), nb, V(W), 2, 256, None) == ALIAS
    assert f(V(W), nb, V(Y), 2, 255, None) == SHAPE


def iq4(w=W, nbytes=None, x=X, y=Y, m=1, n=2, k=256):
    nbytes = q.iq4_xs_bytes(n, k) if nbytes is None else nbytes
    return L.qmv_iq4_xs(V(w), nbytes, V(x), V(y), m, n, k, None)


def test_iq4_xs_validation():
    assert iq4(w=0) == NULL and iq4(x=0) == NULL and iq4(y=0) == NULL
    assert iq4(m=0) == RANGE and iq4(m=5) == RANGE
    assert iq4(n=0) == SHAPE and iq4(k=0) == SHAPE and iq4(k=255) == SHAPE and iq4(k=384) == SHAPE
    assert iq4(w=W + 4) == ALIGN and iq4(x=X + 8) == ALIGN and iq4(y=Y + 2) == ALIGN
    assert iq4(w=W + 8) != ALIGN                          # 136-byte blocks: 8-byte alignment suffices
    assert iq4(m=4, k=19200) == RANGE and iq4(m=3, k=19200) != RANGE   # LDS: m=4 stops at k = 18944
    assert iq4(y=W + 64) == ALIAS
    full = q.iq4_xs_bytes(2, 512)
    for b in list(range(full)) + [full + 1, full + 136]:
        assert iq4(nbytes=b, k=512) == SIZE, b
    nb = q.iq4_xs_bytes(2, 256)
    fn = L.qmv_dequant_iq4_xs_f32
    assert fn(V(0), nb, V(Y), 2, 256, None) == NULL and fn(V(W), nb - 1, V(Y), 2, 256, None) == SIZE
    assert fn(V(W), nb, V(Y + 8), 2, 256, None) == ALIGN and fn(V(W), nb, V(W), 2, 256, None) == ALIAS


def test_q8_0_validation():
    assert q80(w=0) == NULL and q80(x=0) == NULL and q80(y=0) == NULL
    assert q80(m=0) == RANGE and q80(m=5) == RANGE
    assert q80(k=48) == SHAPE and q80(n=-1) == SHAPE
    assert q80(w=W + 2) == ALIGN and q80(x=X + 4) == ALIGN
    assert q80(m=4, k=10272) == RANGE
    assert q80(y=W + 4) == ALIAS
    full = q.q8_0_bytes(2, 64)
    for b in list(range(full)) + [full + 1]:
        assert q80(nbytes=b) == SIZE, b


def test_dequant_validation():
    nb = q.q4_k_bytes(2, 256)
    for fn in (L.qmv_dequant_q4_k_f32, L.qmv_dequant_q4_k_bf16):
        assert fn(V(0), nb, V(Y), 2, 256, None) == NULL
        assert fn(V(W), nb, V(0), 2, 256, None) == NULL
        assert fn(V(W), nb - 1, V(Y), 2, 256, None) == SIZE
        assert fn(V(W), nb, V(Y + 4), 2, 256, None) == ALIGN
        assert fn(V(W), nb, V(W), 2, 256, None) == ALIAS
        assert fn(V(W), nb, V(Y), 2, 100, None) == SHAPE
    nb8 = q.q8_0_bytes(2, 64)
    assert L.qmv_dequant_q8_0_f32(V(W), nb8 - 34, V(Y), 2, 64, None) == SIZE
    assert L.qmv_dequant_q8_0_f32(V(W), nb8, V(Y + 8), 2, 64, None) == ALIGN


def test_prefill_validation():
    nb = q.q4_k_bytes(4, 512)
    f = L.qmm_q4_k_prefill
    assert f(V(W), nb, V(X), V(Y), 0, 4, 512, None, 0, None) == RANGE
    assert f(V(W), nb, V(0), V(Y), 8, 4, 512, None, 0, None) == NULL
    assert f(V(W), nb + 144, V(X), V(Y), 8, 4, 512, None, 0, None) == SIZE
    assert f(V(W), nb, V(X), V(Y + 4), 8, 4, 512, None, 0, None) == ALIGN
    assert f(V(W), nb, V(X), V(X + 16), 8, 4, 512, None, 0, None) == ALIAS
    assert f(V(W), nb, V(X), V(Y), 8, 4, 512, V(WS + 128), 1 << 20, None) == ALIGN   # workspace alignment
    assert f(V(W), nb, V(X), V(Y), 8, 4, 512, V(X), 1 << 20, None) == ALIAS          # workspace over an input
    # the K-split plan is a function of the shape alone (256 workgroup slots, 256 x 128
    # tiles, parts of whole 256-value K blocks), here derived by hand:
    #  512 x 17408 x 5120: 2 x 136 = 272 tiles = 256 whole + 16 split; 20 K blocks, at most
    #    256 / 16 = 16 parts -> parts of ceil(20 / 16) = 2 blocks -> 10 parts: 10 * 16 * 128 KiB
    #  512 x 5120 x 17408: 2 x 40 = 80 tiles, all split; 68 K blocks, at most 256 / 80 = 3
    #    parts -> parts of ceil(68 / 3) = 23 blocks -> 3 parts: 3 * 80 * 128 KiB
    #  256 x 32768 x 5120: exactly 256 tiles, none split; 1 x 16 x 256: one K block, no split
    assert L.qmm_q4_k_prefill_workspace(512, 17408, 5120) == 10 * 16 * 256 * 128 * 4
    assert L.qmm_q4_k_prefill_workspace(512, 5120, 17408) == 3 * 80 * 256 * 128 * 4
    assert L.qmm_q4_k_prefill_workspace(256, 32768, 5120) == 0
    assert L.qmm_q4_k_prefill_workspace(1, 16, 256) == 0
    assert L.qmm_q4_k_prefill_workspace(64, 128, 1024) == 4 * 1 * 256 * 128 * 4   # 1 tile in 4 parts of 1 block
    assert L.qmm_q4_k_prefill_workspace(0, 16, 256) == 0 and L.qmm_q4_k_prefill_workspace(1, 16, 100) == 0
    # a shape whose plan splits is refused without its workspace, or with too little
    nbp = q.q4_k_bytes(128, 1024)
    assert f(V(W), nbp, V(X), V(Y), 64, 128, 1024, None, 0, None) == WORKSPACE
    assert f(V(W), nbp, V(X), V(Y), 64, 128, 1024, V(WS), 4 * 131072 - 1, None) == WORKSPACE
    # the 32-bit activation granule index: m * k / 8 must stay below 2^32 (and the tiles fit an int)
    big_k = 1 << 20
    nbk = q.q4_k_bytes(4, big_k)
    assert f(V(W), nbk, V(X), V(Y), (1 << 15) + 1, 4, big_k, None, 0, None) == RANGE
    assert L.qmm_q4_k_prefill_workspace((1 << 15) + 1, 4, big_k) == 0


def moe(**kw):
    a = dict(wg=W, wu=W + (1 << 28), wd=W + (2 << 28), bank=None, logits=X, x=X + (1 << 20), y=Y,
             ids=Y + (1 << 20), wts=Y + (2 << 20), pairs=Y + (3 << 20), ws=WS, ws_bytes=None,
             t=1, h=256, f=256, e=8, k=2)
    a.update(kw)
    bank = a["e"] * a["f"] * (a["h"] // 256) * 144 if a["bank"] is None else a["bank"]
    need = L.qmv_q4_k_moe_workspace(a["t"], a["h"], a["f"], a["e"], a["k"])
    ws_bytes = need if a["ws_bytes"] is None else a["ws_bytes"]
    return L.qmv_q4_k_moe(V(a["wg"]), V(a["wu"]), V(a["wd"]), bank, V(a["logits"]), V(a["x"]), V(a["y"]),
                          V(a["ids"]), V(a["wts"]), V(a["pairs"]), V(a["ws"]), ws_bytes,
                          a["t"], a["h"], a["f"], a["e"], a["k"], None)


def test_moe_validation():
    assert L.qmv_q4_k_moe_workspace(1, 2048, 768, 128, 8) > 0
    assert L.qmv_q4_k_moe_workspace(0, 2048, 768, 128, 8) == 0
    assert L.qmv_q4_k_moe_workspace(5, 2048, 768, 128, 8) == 0
    assert L.qmv_q4_k_moe_workspace(1, 2048, 768, 128, 9) == 0
    assert moe(wg=0) == NULL and moe(logits=0) == NULL and moe(y=0) == NULL
    assert moe(t=0) == RANGE and moe(t=5) == RANGE and moe(k=0) == RANGE and moe(k=9, e=16) == RANGE
    assert moe(k=4, e=3) == RANGE and moe(e=257) == RANGE
    assert moe(h=300) == SHAPE and moe(f=0) == SHAPE
    assert moe(t=4, k=8, e=16, f=1280) == RANGE          # 32 pairs' h exceed the LDS stage
    assert moe(t=4, h=18432) == RANGE                     # 4 tokens' activations exceed it
    assert moe(bank=8 * 256 * 144 - 1) == SIZE and moe(bank=8 * 256 * 144 + 144) == SIZE
    assert moe(wd=W + (2 << 28) + 8) == ALIGN and moe(ws=WS + 128) == ALIGN and moe(x=X + 2) == ALIGN
    assert moe(ws=0) == WORKSPACE and moe(ws_bytes=16) == WORKSPACE
    assert moe(y=W + 1024) == ALIAS                       # output inside the gate bank
    assert moe(ws=Y) == ALIAS                             # workspace over the output
    assert moe(pairs=Y + (1 << 20)) == ALIAS              # two outputs overlap


def moe_prefill(**kw):
    a = dict(wg=W, wu=W + (1 << 28), wd=W + (2 << 28), bank=None, logits=X, x=X + (1 << 20), y=Y,
             ids=Y + (1 << 20), wts=Y + (2 << 20), ws=WS, ws_bytes=None, t=9, h=256, f=256, e=8, k=2)
    a.update(kw)
    bank = a["e"] * a["f"] * (a["h"] // 256) * 144 if a["bank"] is None else a["bank"]
    need = L.qmv_q4_k_moe_prefill_workspace(a["t"], a["h"], a["f"], a["e"], a["k"])
    ws_bytes = need if a["ws_bytes"] is None else a["ws_bytes"]
    return L.qmv_q4_k_moe_prefill(V(a["wg"]), V(a["wu"]), V(a["wd"]), bank, V(a["logits"]), V(a["x"]), V(a["y"]),
                                  V(a["ids"]), V(a["wts"]), V(a["ws"]), ws_bytes,
                                  a["t"], a["h"], a["f"], a["e"], a["k"], None)


def test_moe_prefill_validation():
    # the workspace holds the routing, the per-expert lists and every pair's h and z
    w512 = L.qmv_q4_k_moe_prefill_workspace(512, 2048, 768, 128, 8)
    assert w512 > 512 * 8 * (768 + 2048) * 4
    assert L.qmv_q4_k_moe_prefill_workspace(1024, 2048, 768, 128, 8) > w512
    assert L.qmv_q4_k_moe_prefill_workspace(0, 2048, 768, 128, 8) == 0
    assert L.qmv_q4_k_moe_prefill_workspace(65537, 2048, 768, 128, 8) == 0
    assert L.qmv_q4_k_moe_prefill_workspace(8, 2048, 768, 128, 9) == 0
    assert moe_prefill(wg=0) == NULL and moe_prefill(logits=0) == NULL and moe_prefill(y=0) == NULL
    assert moe_prefill(t=0) == RANGE and moe_prefill(t=65537) == RANGE and moe_prefill(k=9, e=16) == RANGE
    assert moe_prefill(h=300) == SHAPE and moe_prefill(f=0) == SHAPE
    assert moe_prefill(h=10240) == RANGE                      # 16 tokens' activations exceed the LDS stage
    # the LDS stage limits: hidden 4608 and ffn 1536 fit, one more super-block of either does not
    assert L.qmv_q4_k_moe_prefill_workspace(1, 4608, 1536, 8, 2) > 0
    assert L.qmv_q4_k_moe_prefill_workspace(1, 4864, 256, 8, 2) == 0
    assert L.qmv_q4_k_moe_prefill_workspace(1, 256, 1792, 8, 2) == 0
    assert moe_prefill(bank=8 * 256 * 144 - 1) == SIZE
    assert moe_prefill(ws=0) == WORKSPACE and moe_prefill(ws_bytes=16) == WORKSPACE
    assert moe_prefill(x=X + 2) == ALIGN and moe_prefill(ws=WS + 128) == ALIGN
    # the aliasing checks cover all t tokens: y of 9 tokens (9 KiB) reaches ids 8 KiB after it
    assert moe_prefill(ids=Y + 8192) == ALIAS
    assert moe_prefill(t=600, y=X + (1 << 20) + 1024) == ALIAS   # y inside the 600 tokens' activations
    assert moe_prefill(ws=Y + 4096) == ALIAS                      # workspace over the output


def test_moe_bank_every_truncated_size_is_an_error():
    bank = 8 * 256 * 144
    for b in range(0, bank, 97):
        assert moe(bank=b) == SIZE, b
    assert moe(bank=bank - 1) == SIZE


def moe_iq4(**kw):
    a = dict(wg=W, wu=W + (1 << 28), wd=W + (2 << 28), bank=None, logits=X, x=X + (1 << 20), y=Y,
             ids=Y + (1 << 20), wts=Y + (2 << 20), pairs=Y + (3 << 20), ws=WS, ws_bytes=None,
             t=1, h=256, f=256, e=8, k=2)
    a.update(kw)
    bank = a["e"] * a["f"] * (a["h"] // 256) * 136 if a["bank"] is None else a["bank"]
    need = L.qmv_iq4_xs_moe_workspace(a["t"], a["h"], a["f"], a["e"], a["k"])
    ws_bytes = need if a["ws_bytes"] is None else a["ws_bytes"]
    return L.qmv_iq4_xs_moe(V(a["wg"]), V(a["wu"]), V(a["wd"]), bank, V(a["logits"]), V(a["x"]), V(a["y"]),
                            V(a["ids"]), V(a["wts"]), V(a["pairs"]), V(a["ws"]), ws_bytes,
                            a["t"], a["h"], a["f"], a["e"], a["k"], None)


def test_iq4_xs_moe_validation():
    assert L.qmv_iq4_xs_moe_workspace(1, 2048, 768, 128, 8) == L.qmv_q4_k_moe_workspace(1, 2048, 768, 128, 8)
    assert L.qmv_iq4_xs_moe_workspace(0, 2048, 768, 128, 8) == 0
    assert L.qmv_iq4_xs_moe_workspace(5, 2048, 768, 128, 8) == 0
    assert L.qmv_iq4_xs_moe_workspace(1, 2048, 768, 128, 9) == 0
    assert moe_iq4(wg=0) == NULL and moe_iq4(logits=0) == NULL and moe_iq4(y=0) == NULL
    assert moe_iq4(t=0) == RANGE and moe_iq4(t=5) == RANGE and moe_iq4(k=0) == RANGE
    assert moe_iq4(k=4, e=3) == RANGE and moe_iq4(e=257) == RANGE
    assert moe_iq4(h=300) == SHAPE and moe_iq4(f=0) == SHAPE
    assert moe_iq4(t=4, k=8, e=16, f=1280) == RANGE      # 32 pairs' h exceed the LDS stage
    assert moe_iq4(t=4, k=8, e=16, f=1024) != RANGE      # ... and fit below it
    assert moe_iq4(t=4, h=20480) == RANGE                 # 4 tokens' activations exceed it
    assert moe_iq4(bank=8 * 256 * 136 - 1) == SIZE and moe_iq4(bank=8 * 256 * 144) == SIZE
    assert moe_iq4(wd=W + (2 << 28) + 4) == ALIGN and moe_iq4(x=X + 8) == ALIGN and moe_iq4(ws=WS + 128) == ALIGN
    assert moe_iq4(ws=0) == WORKSPACE and moe_iq4(ws_bytes=16) == WORKSPACE
    assert moe_iq4(y=W + 1024) == ALIAS
    assert moe_iq4(ws=Y) == ALIAS
    assert moe_iq4(pairs=Y + (1 << 20)) == ALIAS


def test_one_hip_runtime_in_the_process():
    # the library must bind to the HIP runtime torch loaded, never load a second one
    import torch  # noqa: F401
    with open("/proc/self/maps") as f:
        paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    real = {os.path.realpath(p) for p in paths}
    assert len(real) == 1, real
