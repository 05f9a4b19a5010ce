"""The file format of tests/c_abi/moe_ep_path (its header comment), written
and read with numpy."""
import os

import numpy as np

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "moe_ep_path")


def program() -> str:
    """The built program; builds it (gcc, about a second) when it is missing."""
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "c_abi_build", os.path.join(os.path.dirname(EXE), "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return EXE


def write_inputs(path, w, srcs, hidden, header=None):
    """srcs: (topk_ids [T, K] int32, topk_weights [T, K] fp32) per source;
    hidden: bf16 bits [T, H] per source. header overrides (T, H, E, K, W,
    max_num_tokens)."""
    hdr = header if header is not None else (w.T, w.H, w.E, w.K, w.W, w.cap)
    with open(path, "wb") as f:
        f.write(np.asarray(hdr, np.int64).tobytes())
        for (ids, wts), h in zip(srcs, hidden):
            f.write(np.ascontiguousarray(ids, np.int32).tobytes())
            f.write(np.ascontiguousarray(wts, np.float32).tobytes())
            f.write(np.ascontiguousarray(h, np.uint16).tobytes())


def read_outputs(path, w):
    raw = np.fromfile(path, np.uint8)
    pos = 0

    def take(dtype, count):
        nonlocal pos
        n = np.dtype(dtype).itemsize * count
        a = raw[pos:pos + n].view(dtype)
        pos += n
        return a

    out = {"send_cnt": [], "token_slot": [], "out": []}
    for _ in range(w.W):
        out["send_cnt"].append(take(np.int32, w.W))
        out["token_slot"].append(take(np.int32, w.T * w.W).reshape(w.T, w.W))
        out["out"].append(take(np.uint16, w.T * w.H).reshape(w.T, w.H))
    ent = take(np.int32, w.e_local * w.W).reshape(w.W, w.e_local)
    out["expert_num_tokens"] = list(ent)
    out["err"] = int(take(np.uint32, 1)[0])
    assert pos == raw.size, (pos, raw.size)
    return out
