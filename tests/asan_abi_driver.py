"""Host-code driver for the AddressSanitizer build of the C ABI (no GPU, no torch).

Run as `python asan_abi_driver.py LIB [--short-counts]` with the ASan runtime
preloaded. It calls every host path of the library: status strings,
workspace sizes for many problems and every stage, moe_plan with counts in
malloc'ed host memory (so a read past the E counts lands in an ASan
redzone), and each entry point's argument checks with arguments that are
rejected before anything is enqueued. Prints "ok <calls>" when every call returned the expected status;
ASan aborts the process on any invalid host memory access. --short-counts
instead hands moe_plan a counts buffer one entry short of E, a caller's
mistake that ASan must report.
"""

import ctypes
import random
import sys

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_expert", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class GemmPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tile", "bm", "bn", "bk", "grid", "k_steps", "max_split",
                                              "min_steps", "split_in_launch")] + \
               [("tiles", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("xcd_rounds", "xcd_leftover", "xcd_split", "split_xcds")]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("route_splits", "route_tokens_per_block", "route_fused_permute",
                                              "permute_form", "gather_in_gemm", "combine_streaming")] + \
               [("gemm", GemmPlan * 2), ("forward_one_launch", ctypes.c_int32)]


def main(path, short_counts=False):
    lib = ctypes.CDLL(path)
    libc = ctypes.CDLL(None)  # the process's malloc: ASan's, with redzones, when its runtime is preloaded
    libc.malloc.restype = ctypes.c_void_p
    libc.malloc.argtypes = [ctypes.c_size_t]
    libc.free.argtypes = [ctypes.c_void_p]
    vp = ctypes.c_void_p
    lib.moe_status_str.restype = ctypes.c_char_p
    calls = 0

    def expect(got, want, what):
        nonlocal calls
        calls += 1
        if got != want:
            raise SystemExit(f"{what}: status {got}, expected {want}")

    for st in range(-1, 7):
        assert lib.moe_status_str(st)
        calls += 1

    if short_counts:
        E = 16
        buf = libc.malloc(4 * (E - 1))
        counts = (ctypes.c_int32 * (E - 1)).from_address(buf)
        for e in range(E - 1):
            counts[e] = 4
        lib.moe_plan(ctypes.byref(Problem(32, 512, E, 2, 1024, 1)), vp(buf), ctypes.byref(Plan()))
        raise SystemExit("a read past the counts went unreported")

    rng = random.Random(5)
    shapes = [(1, 64, 1, 1, 64, 1), (64, 128, 8, 2, 256, 0), (4096, 2048, 8, 2, 8192, 1),
              (16384, 7168, 256, 8, 2048, 1), (777, 320, 12, 3, 448, 1), (5, 512, 16, 2, 1024, 1)]
    for _ in range(60):
        E = rng.randint(1, 256)
        shapes.append((rng.randint(1, 70000), 64 * rng.randint(1, 64), E, rng.randint(1, min(E, 8)),
                       64 * rng.randint(1, 64), rng.randint(0, 1)))
    size = ctypes.c_size_t(0)
    for T, d, E, k, de, dt in shapes:
        p = Problem(T, d, E, k, de, dt)
        for stage in range(5):
            r = lib.moe_workspace_size(ctypes.byref(p), stage, ctypes.byref(size))
            expect(r in (OK, UNSUPPORTED), True, f"moe_workspace_size {T, d, E, k, de, dt} stage {stage}")
        plan = Plan()
        expect(lib.moe_plan(ctypes.byref(p), None, ctypes.byref(plan)), OK, "moe_plan")
        # counts in malloc'ed memory of exactly E int32: balanced, random, all on one expert
        buf = libc.malloc(4 * E)
        counts = (ctypes.c_int32 * E).from_address(buf)
        R = T * k
        for mode in range(3):
            if mode == 0:
                vals = [R // E + (1 if e < R % E else 0) for e in range(E)]
            elif mode == 1:
                cut = sorted(rng.randint(0, R) for _ in range(E - 1))
                vals = [b - a for a, b in zip([0] + cut, cut + [R])]
            else:
                vals = [0] * E
                vals[rng.randrange(E)] = R
            for e in range(E):
                counts[e] = vals[e]
            expect(lib.moe_plan(ctypes.byref(p), vp(buf), ctypes.byref(plan)), OK, "moe_plan counts")
        counts[E - 1] = -1
        expect(lib.moe_plan(ctypes.byref(p), vp(buf), ctypes.byref(plan)), INVALID, "moe_plan negative count")
        libc.free(buf)

    # every entry point rejects before enqueueing: bad problems, NULL or misaligned
    # pointers, a workspace that is too small
    A, A2, MIS = vp(0x10000), vp(0x20000), vp(0x10008)
    good = Problem(64, 128, 8, 2, 256, 1)
    bad = [Problem(0, 128, 8, 2, 256, 1), Problem(64, 96, 8, 2, 256, 1), Problem(64, 128, 300, 2, 256, 1),
           Problem(64, 128, 8, 9, 256, 1), Problem(64, 128, 8, 2, 256, 7)]
    small = ctypes.c_size_t(16)
    for p in bad:
        pr = ctypes.byref(p)
        want = {0: INVALID, 96: UNSUPPORTED}.get(p.T if p.T == 0 else p.d_model)
        for r in (lib.moe_route(pr, A, A, None, None, A, A, None),
                  lib.moe_route_ws(pr, A, A, None, None, A, A, A2, ctypes.c_size_t(1 << 30), None),
                  lib.moe_permute(pr, A, A, A, A, A, A, A, A2, ctypes.c_size_t(1 << 30), None),
                  lib.moe_permute_index(pr, A, A, A, A, A, A2, ctypes.c_size_t(1 << 30), None),
                  lib.moe_grouped_ffn(pr, A, A, A, A, A, A2, ctypes.c_size_t(1 << 30), None),
                  lib.moe_combine(pr, A, A, A, A, None),
                  lib.moe_forward(pr, A, A, None, A, A, A, A2, ctypes.c_size_t(1 << 30), None)):
            expect(r != OK, True, f"bad problem {p.T, p.d_model, p.E, p.k, p.dtype}")
            if want is not None:
                expect(r, want, f"bad problem status {p.T, p.d_model}")
    pr = ctypes.byref(good)
    expect(lib.moe_route(pr, None, A, None, None, A, A, None), INVALID, "route NULL x")
    expect(lib.moe_route(pr, MIS, A, None, None, A, A, None), INVALID, "route misaligned x")
    expect(lib.moe_permute(pr, A, A, A, A, A, A, A, A2, small, None), WS_SMALL, "permute small ws")
    expect(lib.moe_permute_index(pr, A, A, A, A, A, A2, small, None), WS_SMALL, "permute_index small ws")
    expect(lib.moe_grouped_ffn(pr, A, A, A, A, A, A2, small, None), WS_SMALL, "ffn small ws")
    expect(lib.moe_grouped_ffn_gather(pr, A, A, A, A, A, A, A2, small, None), WS_SMALL, "ffn_gather small ws")
    expect(lib.moe_forward(pr, A, A, None, A, A, A, A2, small, None), WS_SMALL, "forward small ws")
    expect(lib.moe_forward_train(pr, A, A, None, A, A, A, A2, small, None), WS_SMALL, "forward_train small ws")
    expect(lib.moe_backward(pr, A, A, A, A, A, A, A, A, A, A, A, A, A2, small, None), WS_SMALL,
           "backward small ws")
    expect(lib.moe_combine(pr, A, A, A, MIS, None), INVALID, "combine misaligned y")
    expect(lib.moe_permute_index_noalloc(pr, None, A, A, A, A, None), INVALID, "noalloc NULL idx")
    big = Problem(1 << 22, 128, 256, 2, 256, 1)
    expect(lib.moe_permute_index_noalloc(ctypes.byref(big), A, A, A, A, A, None), WS_SMALL, "noalloc too large")
    print(f"ok {calls}")


if __name__ == "__main__":
    main(sys.argv[1], "--short-counts" in sys.argv[2:])
