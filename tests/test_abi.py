"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host before touching the GPU (CPU only: no compute call)."""
import ctypes
import os
import re
import subprocess

import pytest

from semi_ar_drafter_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from semi_ar_drafter_amd import build_lib
        build_lib.build(verbose=False)
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"dspark_markov_draft", "dspark_schedule", "dspark_verify"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dspark_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


# fake, suitably aligned device addresses: never dereferenced by failing calls
P = ctypes.c_void_p(0x10000)
NULL = ctypes.c_void_p(0)


def draft(lib, B=4, gamma=4, V=1024, r=32, d=16, dtype=1, mode=0, ws=P, ws_bytes=None, **over):
    ptrs = dict(anchor=P, U=P, h=P, W1=P, W2=P, conf_w=P, sts_T=P, tokens=P, logit=P, conf=P, surv=P)
    ptrs.update(over)
    if ws_bytes is None:
        ws_bytes = lib.dspark_draft_workspace_bytes(max(B, 1), max(gamma, 1), V, r)
    return lib.dspark_markov_draft(B, gamma, V, r, d, dtype, ptrs["anchor"], ptrs["U"], ptrs["h"], ptrs["W1"],
                                   ptrs["W2"], ptrs["conf_w"], ctypes.c_float(1.0), ptrs["sts_T"], mode,
                                   ctypes.c_uint64(0), ptrs["tokens"], ptrs["logit"], ptrs["conf"], ptrs["surv"],
                                   ws, ctypes.c_size_t(ws_bytes), NULL)


def test_draft_validation(lib):
    assert draft(lib, B=-1) == INVALID
    assert draft(lib, V=-3) == INVALID
    assert draft(lib, dtype=7) == INVALID
    assert draft(lib, mode=3) == INVALID
    assert draft(lib, V=0) == INVALID
    for name in ("anchor", "U", "W1", "W2", "conf_w", "sts_T", "tokens", "logit", "conf", "surv", "h"):
        assert draft(lib, **{name: NULL}) == INVALID, name
    assert draft(lib, gamma=65) == UNSUPPORTED
    assert draft(lib, d=70000) == UNSUPPORTED
    assert draft(lib, r=48) == UNSUPPORTED                # bf16 needs r in {32, 64, 128, 256}
    assert draft(lib, dtype=0, r=256) == UNSUPPORTED      # fp32 needs r in {16, 32, 64}
    assert draft(lib, W1=ctypes.c_void_p(0x10008)) == INVALID   # W1 rows read 16 bytes at a time
    assert draft(lib, ws=NULL) == WORKSPACE
    assert draft(lib, ws_bytes=100) == WORKSPACE
    assert draft(lib, ws=ctypes.c_void_p(0x10040)) == WORKSPACE  # not 256-byte aligned
    assert lib.dspark_last_error().decode() != ""
    # empty batches are valid no-ops and need no pointers at all
    assert draft(lib, B=0, anchor=NULL, U=NULL, ws=NULL, ws_bytes=0) == OK
    assert draft(lib, gamma=0, anchor=NULL, U=NULL, ws=NULL, ws_bytes=0) == OK


def rnn(lib, B=4, gamma=4, V=1024, r=32, d=16, dtype=1, mode=0, ws=P, ws_bytes=None, decay=P, **over):
    ptrs = dict(anchor=P, U=P, h=P, W1=P, W2=P, conf_w=P, sts_T=P, tokens=P, logit=P, conf=P, surv=P)
    ptrs.update(over)
    if ws_bytes is None:
        ws_bytes = lib.dspark_rnn_draft_workspace_bytes(max(B, 1), max(gamma, 1), V, r)
    return lib.dspark_rnn_draft(B, gamma, V, r, d, dtype, ptrs["anchor"], ptrs["U"], ptrs["h"], ptrs["W1"],
                                ptrs["W2"], decay, ptrs["conf_w"], ctypes.c_float(1.0), ptrs["sts_T"], mode,
                                ctypes.c_uint64(0), ptrs["tokens"], ptrs["logit"], ptrs["conf"], ptrs["surv"],
                                ws, ctypes.c_size_t(ws_bytes), NULL)


def test_rnn_draft_validation(lib):
    assert rnn(lib, dtype=0) == UNSUPPORTED                  # the RNN head is built for bf16 storage
    assert rnn(lib, dtype=7) == INVALID
    assert rnn(lib, decay=NULL) == INVALID
    assert rnn(lib, decay=ctypes.c_void_p(0x10002)) == INVALID
    for name in ("anchor", "U", "W1", "W2", "conf_w", "sts_T", "tokens", "logit", "conf", "surv"):
        assert rnn(lib, **{name: NULL}) == INVALID, name
    assert rnn(lib, r=48) == UNSUPPORTED
    assert rnn(lib, gamma=65) == UNSUPPORTED
    markov_bytes = lib.dspark_draft_workspace_bytes(4, 4, 1024, 32)
    assert rnn(lib, ws_bytes=markov_bytes) == WORKSPACE      # the state section is missing
    assert "dspark_rnn_draft_workspace_bytes" in lib.dspark_last_error().decode()
    assert rnn(lib, B=0, anchor=NULL, U=NULL, ws=NULL, ws_bytes=0) == OK


def test_rnn_workspace_size(lib):
    assert lib.dspark_rnn_draft_workspace_bytes(0, 16, 151936, 256) == 0
    assert lib.dspark_rnn_draft_workspace_bytes(256, 16, 151936, 0) == 0
    m = lib.dspark_draft_workspace_bytes(256, 16, 151936, 256)
    a = lib.dspark_rnn_draft_workspace_bytes(256, 16, 151936, 256)
    assert a % 256 == 0 and a >= m + 2 * 256 * 256 * 2


def test_gumbel_from_words_validation(lib):
    assert lib.dspark_gumbel_from_words(-1, P, P, NULL) == INVALID
    assert lib.dspark_gumbel_from_words(4, NULL, P, NULL) == INVALID
    assert lib.dspark_gumbel_from_words(4, P, NULL, NULL) == INVALID
    assert lib.dspark_gumbel_from_words(4, ctypes.c_void_p(0x10002), P, NULL) == INVALID
    assert lib.dspark_gumbel_from_words(0, NULL, NULL, NULL) == OK


def test_workspace_size(lib):
    assert lib.dspark_draft_workspace_bytes(0, 16, 151936, 256) == 0
    a = lib.dspark_draft_workspace_bytes(256, 16, 151936, 256)
    b = lib.dspark_draft_workspace_bytes(512, 16, 151936, 256)
    assert a % 256 == 0 and b % 256 == 0 and b > a > 256 * 16 * 8


def test_small_batch_workspace_holds_the_winner_keys(lib):
    """Batches of at most 16 requests also carve every workgroup's winner key
    (8 bytes) and Gumbel logit (4 bytes) per position and request, for up to
    512 workgroups; larger batches do not."""
    for B, gamma in ((1, 8), (16, 64)):
        n = lib.dspark_draft_workspace_bytes(B, gamma, 151936, 256)
        assert n % 256 == 0 and n >= gamma * B * 512 * 12
        assert n <= 8 << 20   # within the allocation-free entry point's scratch
    assert lib.dspark_draft_workspace_bytes(17, 64, 151936, 256) < 17 * 64 * 512 * 12


def sched(lib, B=4, gamma=4, n_min=4, n_count=17, surv=P, t=P, lens=P, m=P, ws=NULL, ws_bytes=0):
    return lib.dspark_schedule(B, gamma, surv, t, n_min, n_count, lens, m, NULL, ws, ctypes.c_size_t(ws_bytes),
                               NULL)


def test_schedule_validation(lib):
    assert sched(lib, B=-1) == INVALID
    assert sched(lib, n_count=0) == INVALID
    assert sched(lib, n_min=5) == INVALID                 # table starts above B
    assert sched(lib, n_min=0, n_count=4) == INVALID      # table ends below B
    assert sched(lib, surv=NULL) == INVALID
    assert sched(lib, t=NULL) == INVALID
    assert sched(lib, lens=NULL) == INVALID
    assert sched(lib, m=NULL) == INVALID
    assert sched(lib, B=1025, gamma=16, n_min=1025, n_count=16401) == UNSUPPORTED
    need = lib.dspark_schedule_workspace_bytes(4, 4)
    assert sched(lib, ws=P, ws_bytes=need - 1) == WORKSPACE
    assert sched(lib, ws=ctypes.c_void_p(0x10080), ws_bytes=need) == WORKSPACE
    assert "workspace" in lib.dspark_last_error().decode()


def test_schedule_workspace_size(lib):
    ws = lib.dspark_schedule_workspace_bytes
    assert ws(0, 16) == 0 and ws(16, 0) == 0 and ws(-1, 4) == 0 and ws(1025, 16) == 0
    # a 2 KiB block of ticket counters, then 16 bytes (sort key, step cost)
    # per entry, in whole rows of 512
    assert ws(256, 16) == 2048 + 4096 * 16
    assert ws(3, 5) == 2048 + 512 * 16 and ws(1024, 16) == 2048 + 16384 * 16
    d = lib.dspark_draft_workspace_bytes(256, 16, 151936, 256)
    assert lib.dspark_serve_workspace_bytes(256, 16, 151936, 256) == d + ws(256, 16)
    assert lib.dspark_serve_workspace_bytes(0, 16, 151936, 256) == 0


def test_verify_validation(lib):
    v = lambda B=4, g=4, tk=P, tg=P, ln=P, a=P, bo=P: lib.dspark_verify(B, g, tk, tg, ln, a, bo, NULL)
    assert v(B=-2) == INVALID
    assert v(g=-1) == INVALID
    assert v(tk=NULL) == INVALID
    assert v(tg=NULL) == INVALID
    assert v(ln=NULL) == INVALID
    assert v(a=NULL) == INVALID
    assert v(bo=NULL) == INVALID
    assert v(B=0, tk=NULL, tg=NULL) == OK


def test_parallel_draft_validation(lib):
    pd = lambda B=2, g=3, V=100, dt=1, U=P, mode=0, tk=P, lo=P: lib.dspark_parallel_draft(
        B, g, V, dt, U, mode, 0, tk, lo, NULL)
    assert pd(B=-1) == 1 and pd(V=-5) == 1
    assert pd(dt=7) == 1 and pd(mode=3) == 1
    assert pd(B=0) == 0 and pd(g=0) == 0            # empty: no-op, nothing launched
    assert pd(V=0) == 1
    assert pd(U=NULL) == 1 and pd(tk=NULL) == 1 and pd(lo=NULL) == 1
    assert pd(V=(1 << 24) + 1) == 2
    assert pd(U=ctypes.c_void_p(0x1001)) == 1       # bf16 element misaligned
    assert lib.dspark_last_error().decode() != ""


def test_sts_fit_validation(lib):
    ws_need = lib.dspark_sts_workspace_bytes(1000, 24, 15)
    assert ws_need >= 256 + 24 * 15 * 8 + 1000 * 8
    assert lib.dspark_sts_workspace_bytes(-1, 24, 15) == 0 and lib.dspark_sts_workspace_bytes(10, 0, 15) == 0
    assert lib.dspark_sts_workspace_bytes(10, 4097, 1) == 0 and lib.dspark_sts_workspace_bytes(10, 2, 257) == 0

    def fit(N=1000, g=4, lo=P, acc=P, grid=P, G=24, M=15, ch=P, T=P, ece=P, ws=P, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = ws_need
        return lib.dspark_sts_fit(N, g, lo, acc, grid, G, M, ch, T, ece, ws, ctypes.c_size_t(ws_bytes), NULL)

    assert fit(N=-1) == INVALID and fit(g=-2) == INVALID and fit(G=-1) == INVALID and fit(M=-3) == INVALID
    assert fit(g=0) == OK                                   # no-op, nothing launched
    assert fit(G=0) == INVALID and fit(M=0) == INVALID
    for k in ("lo", "acc", "grid", "ch", "T", "ece"):
        assert fit(**{k: NULL}) == INVALID, k
    assert fit(G=4097, ws_bytes=1 << 30) == UNSUPPORTED
    assert fit(M=257, G=2, ws_bytes=1 << 30) == UNSUPPORTED
    assert fit(G=1024, M=9, ws_bytes=1 << 30) == UNSUPPORTED   # histogram over 8192 entries
    assert fit(N=(1 << 24) + 1, ws_bytes=1 << 40) == UNSUPPORTED
    assert fit(N=1 << 24, g=200, ws_bytes=1 << 40) == UNSUPPORTED   # N * gamma >= 2^31
    assert fit(lo=ctypes.c_void_p(0x10002)) == INVALID
    assert fit(ece=ctypes.c_void_p(0x10004)) == INVALID
    assert fit(ws=NULL) == WORKSPACE and fit(ws_bytes=ws_need - 1) == WORKSPACE
    assert fit(ws=ctypes.c_void_p(0x10080)) == WORKSPACE
    assert "workspace" in lib.dspark_last_error().decode()


def test_schedule_threshold_validation(lib):
    st = lambda B=4, g=4, surv=P, tau=0.5, lens=P, m=P: lib.dspark_schedule_threshold(
        B, g, surv, ctypes.c_float(tau), lens, m, NULL)
    assert st(B=-1) == INVALID and st(g=-1) == INVALID
    assert st(m=NULL) == INVALID and st(lens=NULL) == INVALID and st(surv=NULL) == INVALID
    assert st(B=1 << 20, g=1 << 12) == UNSUPPORTED


def test_serve_validation(lib):
    ws_need = lib.dspark_serve_workspace_bytes(4, 4, 1024, 32)
    draft_need = lib.dspark_draft_workspace_bytes(4, 4, 1024, 32)

    def serve(iters=3, B=4, g=4, V=1024, r=32, d=16, dt=1, policy=0, n_min=4, n_count=17, ws=P, ws_bytes=None,
              mode=0, **over):
        ptr = dict(anchor=P, U=P, h=P, W1=P, W2=P, conf_w=P, sts_T=P, target=P, t_step=P, tokens=P, logit=P,
                   conf=P, surv=P, lens=P, accepted=P, bonus=P, m=P)
        ptr.update(over)
        return lib.dspark_serve(iters, B, g, V, r, d, dt, ptr["anchor"], ptr["U"], ptr["h"], ptr["W1"], ptr["W2"],
                                ptr["conf_w"], ctypes.c_float(1.0), ptr["sts_T"], mode, 0, ptr["target"],
                                ptr["t_step"], n_min, n_count, policy, ctypes.c_float(0.5), ptr["tokens"],
                                ptr["logit"], ptr["conf"], ptr["surv"], ptr["lens"], ptr["accepted"], ptr["bonus"],
                                ptr["m"], ws, ctypes.c_size_t(ws_need if ws_bytes is None else ws_bytes), NULL)

    assert serve(iters=-1) == INVALID and serve(policy=7) == INVALID and serve(B=-2) == INVALID
    assert serve(iters=0) == OK and serve(B=0) == OK and serve(g=0) == OK      # no-ops: nothing launched
    for k in ("target", "lens", "accepted", "bonus", "m", "t_step"):
        assert serve(**{k: NULL}) == INVALID, k
    assert serve(n_count=0) == INVALID
    assert serve(n_min=5) == INVALID and serve(n_min=1, n_count=3) == INVALID   # table must cover n = B
    assert serve(B=4096, g=8, n_count=40000, ws_bytes=1 << 40) == UNSUPPORTED  # global policy: B * gamma > 16384
    # the draft arguments are checked by iteration 0 before anything is enqueued
    assert serve(anchor=NULL) == INVALID and serve(W1=ctypes.c_void_p(0x10008)) == INVALID
    assert serve(ws=NULL) == WORKSPACE and serve(ws_bytes=ws_need - 1) == WORKSPACE
    assert serve(ws_bytes=draft_need) == WORKSPACE          # no room for the scheduler's part
    assert serve(ws_bytes=draft_need - 1) == WORKSPACE
    assert serve(dt=5) == INVALID and serve(mode=4) == INVALID
    assert lib.dspark_last_error().decode() != ""


def test_step_validation(lib):
    need = lib.dspark_step_workspace_bytes(4, 4, 1024, 32)
    assert need == lib.dspark_serve_workspace_bytes(4, 4, 1024, 32) > lib.dspark_draft_workspace_bytes(4, 4, 1024, 32)

    def step(B=4, g=4, V=1024, r=32, d=16, dt=1, n_min=4, n_count=17, ws=P, ws_bytes=None, mode=0, **over):
        ptr = dict(anchor=P, U=P, h=P, W1=P, W2=P, conf_w=P, sts_T=P, target=P, t_step=P, tokens=P, logit=P,
                   conf=P, surv=P, lens=P, m=P, accepted=P, bonus=P)
        ptr.update(over)
        return lib.dspark_step(B, g, V, r, d, dt, ptr["anchor"], ptr["U"], ptr["h"], ptr["W1"], ptr["W2"],
                               ptr["conf_w"], ctypes.c_float(1.0), ptr["sts_T"], mode, 0, ptr["target"],
                               ptr["t_step"], n_min, n_count, ptr["tokens"], ptr["logit"], ptr["conf"], ptr["surv"],
                               ptr["lens"], ptr["m"], ptr["accepted"], ptr["bonus"], ws,
                               ctypes.c_size_t(need if ws_bytes is None else ws_bytes), NULL)

    assert step(B=-1) == INVALID and step(n_count=0) == INVALID
    assert step(B=0) == OK                                   # no-op, nothing launched
    for k in ("target", "t_step", "lens", "m", "accepted", "bonus"):
        assert step(**{k: NULL}) == INVALID, k
    assert step(n_min=5) == INVALID and step(n_min=0, n_count=4) == INVALID
    assert step(B=4097, g=4, n_min=4097, n_count=16389, ws_bytes=1 << 40) == UNSUPPORTED   # B * gamma > 16384
    assert step(ws_bytes=lib.dspark_draft_workspace_bytes(4, 4, 1024, 32)) == WORKSPACE   # no room for the scheduler
    assert step(ws=NULL) == WORKSPACE
    assert step(anchor=NULL) == INVALID and step(dt=5) == INVALID and step(mode=3) == INVALID
    assert lib.dspark_last_error().decode() != ""


def test_draft_launch_mode_setting(lib):
    assert lib.dspark_get_draft_launch() == 0                 # cooperative by default
    assert lib.dspark_set_draft_launch(1) == OK and lib.dspark_get_draft_launch() == 1
    assert lib.dspark_set_draft_launch(5) == INVALID and lib.dspark_get_draft_launch() == 1
    assert lib.dspark_set_draft_launch(0) == OK and lib.dspark_get_draft_launch() == 0


def test_status_strings(lib):
    for s in range(5):
        assert lib.dspark_status_string(s).decode()
    assert lib.dspark_status_string(99).decode() == "unknown status"


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load(str(tmp_path / "missing.so"))


def test_workspace_cache_is_per_device_and_stream(monkeypatch):
    """The binding's library-owned workspace is cached per (device, stream):
    calls on one stream reuse it (growing it when a larger one is needed),
    calls on another stream or device get their own, each zero-filled on the
    stream that will use it.  Exercised with a stand-in for torch's device
    API (no GPU needed)."""
    import contextlib

    class Stream:
        def __init__(self, handle):
            self.cuda_stream = handle

    made = []

    zeroed = []

    class Buf:
        def __init__(self, n, device, stream):
            self.n, self.device, self.stream = n, device, stream

        def numel(self):
            return self.n

        def zero_(self):
            assert Cuda.active is not None, "the re-fill must be enqueued on the caller's stream"
            zeroed.append((self, Cuda.active.cuda_stream))
            return self

    class Cuda:
        current = {0: Stream(0x100), 1: Stream(0x200)}
        active = None

        @staticmethod
        def current_device():
            return 0

        @staticmethod
        def current_stream(index=None):
            return Cuda.current[0 if index is None else index]

        @staticmethod
        @contextlib.contextmanager
        def stream(s):
            prev, Cuda.active = Cuda.active, s
            yield
            Cuda.active = prev

    class Device:
        def __init__(self, index):
            self.index = index

    class Torch:
        cuda = Cuda
        uint8 = "uint8"

        @staticmethod
        def zeros(n, dtype=None, device=None):
            assert Cuda.active is not None, "zero fill must be enqueued on the caller's stream"
            b = Buf(n, device.index, Cuda.active.cuda_stream)
            made.append(b)
            return b

    monkeypatch.setattr(binding, "_torch", lambda: Torch)
    monkeypatch.setattr(binding, "_ws_cache", {})
    d0, d1 = Device(0), Device(1)
    a = binding._workspace(1000, d0)
    assert a.stream == 0x100 and a.device == 0
    assert binding._workspace(500, d0) is a                 # same stream: reused
    big = binding._workspace(5000, d0)                      # larger: replaced on the same stream
    assert big is not a and big.n == 5000 and big.stream == 0x100
    assert binding._workspace(100, d0) is big
    Cuda.current[0] = Stream(0x300)                         # another stream on device 0
    c = binding._workspace(100, d0)
    assert c is not big and c.stream == 0x300
    e = binding._workspace(100, d1)                         # device 1's current stream
    assert e.device == 1 and e.stream == 0x200
    s = binding._workspace(100, d0, kind="sts")             # another kind, same stream
    assert s is not c
    assert len(made) == 5
    assert binding._workspace_key("draft", 0, 0x100) != binding._workspace_key("draft", 0, 0x300)
    # the zero-required parts move with the shape: a change of layout re-fills the reused buffer
    f = binding._workspace(100, d0, "step", (96, 6))
    assert binding._workspace(100, d0, "step", (96, 6)) is f and not zeroed      # same shape: as left
    assert binding._workspace(90, d0, "step", (40, 16)) is f and zeroed == [(f, 0x300)]
    assert binding._workspace(90, d0, "step", (40, 16)) is f and len(zeroed) == 1
