"""Successful calls of every entry point through the sanitizer build.

TEST INFRASTRUCTURE, run by tests/test_host_sanitized.py in a child process
whose libflce is the CPU build of the host layer (g++ with AddressSanitizer
and UndefinedBehaviorSanitizer) over stub launchers: every call below passes
the argument checks, so the chunk loops, workspace layouts and offset
arithmetic run for real, and each stub launch checks that the byte ranges
its kernel would touch lie inside the buffers registered here.  Buffers are
never dereferenced: they are disjoint address ranges 2^44 bytes apart.
"""

import ctypes
import itertools
import sys

import linear_cross_entropy_06_amd._lib as L

BF16, F32 = 0, 1
GAP = 1 << 44


def main(lib_path: str) -> int:
    L.LIB_PATH = lib_path
    lib = L.load()
    lib.flce_stub_add_buffer.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.flce_stub_violations.restype = ctypes.c_int64
    lib.flce_stub_launches.restype = ctypes.c_int64
    lib.flce_stub_last_violation.restype = ctypes.c_char_p
    calls = 0

    def bufs(**sizes):
        lib.flce_stub_reset()
        out = {}
        for i, (name, n) in enumerate(sizes.items()):
            out[name] = (i + 1) * GAP
            lib.flce_stub_add_buffer(out[name], max(int(n), 1))
        return out

    def ok(status, what):
        nonlocal calls
        calls += 1
        v = lib.flce_stub_violations()
        if status != 0 or v != 0:
            print(f"FAIL {what}: status {status}, {v} violations: "
                  f"{lib.flce_stub_last_violation().decode()}", flush=True)
            return False
        return True

    good = True
    shapes = [(1, 64, 8, 1), (3, 8, 5, 2), (17, 24, 1000, 7), (300, 128, 1000, 128),
              (300, 136, 523, 256), (513, 264, 1000, 257), (1024, 512, 8192, 384),
              (2048, 1024, 32000, 512), (2048, 4096, 32000, 2048), (8192, 4096, 128256, 4096),
              (8100, 4096, 128256, 4096), (8192, 4096, 128256, 1024),
              (8192, 3584, 256000, 4096), (16384, 4096, 128256, 4096), (64, 64, 40000, 64),
              (7, 128, 1000, 3), (16, 64, (1 << 22) + 64, 4)]
    # the seeded shapes of the GPU parity sweep as well
    sys.path.insert(0, "tests")
    from parity_util import random_shapes
    shapes += sorted({(N, H, V, C) for N, H, V, C, _ in random_shapes()})
    for (N, H, V, C), dt in itertools.product(shapes, (BF16, F32)):
        es = 2 if dt == BF16 else 4
        need = lib.flce_workspace_bytes(N, H, V, C, dt)
        for entry in ("flce_fwd_bwd", "flce_fwd_bwd_accumulate"):
            b = bufs(h=N * H * es, W=V * H * es, t=N * 4, loss=4, gh=N * H * es, gW=V * H * 4,
                     ws=need)
            st = getattr(lib, entry)(b["h"], b["W"], b["t"], N, H, V, C, b["loss"], b["gh"],
                                     b["gW"], b["ws"], need, dt, None)
            good &= ok(st, f"{entry} {(N, H, V, C, dt)}")
        n_ev = 2 * lib.flce_launch_count(N, C)
        b = bufs(h=N * H * es, W=V * H * es, t=N * 4, loss=4, gh=N * H * es, gW=V * H * 4, ws=need)
        ev = (ctypes.c_void_p * n_ev)()
        st = lib.flce_fwd_bwd_timed(b["h"], b["W"], b["t"], N, H, V, C, b["loss"], b["gh"],
                                    b["gW"], b["ws"], need, dt, None, ev, n_ev)
        good &= ok(st, f"flce_fwd_bwd_timed {(N, H, V, C, dt)}")
        rneed = lib.flce_rmsnorm_workspace_bytes(N, H, V, C, dt)
        b = bufs(x=N * H * es, g=H * es, W=V * H * es, t=N * 4, loss=4, gx=N * H * es,
                 gg=H * 4, gW=V * H * 4, ws=rneed)
        st = lib.flce_fwd_bwd_rmsnorm(b["x"], b["g"], ctypes.c_float(1e-6), b["W"], b["t"], N,
                                      H, V, C, b["loss"], b["gx"], b["gg"], b["gW"], b["ws"],
                                      rneed, dt, None)
        good &= ok(st, f"flce_fwd_bwd_rmsnorm {(N, H, V, C, dt)}")
        if need <= L.NOALLOC_SCRATCH_BYTES:
            b = bufs(h=N * H * es, W=V * H * es, t=N * 4, loss=4, gh=N * H * es, gW=V * H * 4)
            st = lib.flce_fwd_bwd_noalloc(b["h"], b["W"], b["t"], N, H, V, C, b["loss"],
                                          b["gh"], b["gW"], dt, None)
            good &= ok(st, f"flce_fwd_bwd_noalloc {(N, H, V, C, dt)}")
    for (N, H, V, vc) in [(4, 64, 128, 128), (300, 128, 1024, 256), (8192, 4096, 128256, 16384),
                          (1024, 3584, 256000, 32768), (5, 64, 640, 10 ** 6)]:
        need = lib.flce_vocab_workspace_bytes(N, H, V, vc, BF16)
        b = bufs(h=N * H * 2, W=V * H * 2, t=N * 4, loss=4, gh=N * H * 2, gW=V * H * 4, ws=need)
        st = lib.flce_fwd_bwd_vocab(b["h"], b["W"], b["t"], N, H, V, vc, b["loss"], b["gh"],
                                    b["gW"], b["ws"], need, BF16, None)
        good &= ok(st, f"flce_fwd_bwd_vocab {(N, H, V, vc)}")
    for (B, T, H, V, cp) in [(1, 1, 64, 256, 1), (3, 50, 128, 1000, 2), (8, 128, 512, 4096, 3),
                             (4, 1024, 4096, 128256, 2), (2, 512, 1024, 32000, 1)]:
        N = 2 * B * T
        need = lib.flce_orpo_workspace_bytes(B, T, H, V, cp, BF16)
        b = bufs(h=N * H * 2, W=V * H * 2, t=N * 4, loss=4, seq=2 * B * 4, gh=N * H * 2,
                 gW=V * H * 4, ws=need)
        st = lib.flce_orpo_fwd_bwd(b["h"], b["W"], b["t"], B, T, H, V, cp, ctypes.c_float(0.1),
                                   b["loss"], b["seq"], b["gh"], b["gW"], b["ws"], need, BF16,
                                   None)
        good &= ok(st, f"flce_orpo_fwd_bwd {(B, T, H, V, cp)}")
    for (rows, V, ld) in [(1, 5, 5), (1024, 128256, 128256), (300, 1000, 1008)]:
        for dt, es in ((BF16, 2), (F32, 4)):
            b = bufs(z=rows * ld * es, t=rows * 4, loss=4, rl=rows * 4)
            st = lib.flce_cross_entropy(b["z"], ld, b["t"], rows, V, b["loss"], b["rl"], dt, None)
            good &= ok(st, f"flce_cross_entropy {(rows, V, ld, dt)}")
    b = bufs(gh=1000 * 2, gW=4000 * 4, s=4)
    good &= ok(lib.flce_scale_grads(b["gh"], 1000, b["gW"], 4000, b["s"], BF16, None), "scale")
    b = bufs(ops=1 << 20, sink=256 * 4 * 4, clocks=256 * 4 * 2 * 8)
    good &= ok(lib.flce_mfma_rate(b["ops"], 1 << 20, 10, 256, b["sink"], b["clocks"], None),
               "mfma_rate")
    print(f"{calls} successful calls checked, {lib.flce_stub_launches()} launches in the last",
          flush=True)
    return 0 if good else 1


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
