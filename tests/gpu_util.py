"""Helpers for the GPU parity tests: host arrays <-> device tensors, error
measures.  Holds no step of the method."""
import numpy as np
import torch

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_any(a: np.ndarray, dtype: str) -> torch.Tensor:
    return dev_bf16(a) if dtype == "bf16" else dev_f32(a)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_i(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are all zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def case_to_device(c):
    """Device tensors of a synth.MoECase (None where absent)."""
    d = {}
    if c.logits is not None:
        d["logits"] = dev_any(c.logits, c.logits_dtype)
    d["x"] = dev_any(c.x, c.x_dtype)
    if c.w_dtype == "mxfp4":
        d["w1"], d["w2"] = dev_u8(c.w1), dev_u8(c.w2)
        d["w1_scale"], d["w2_scale"] = dev_u8(c.w1_scale), dev_u8(c.w2_scale)
    elif c.w1 is not None:
        d["w1"], d["w2"] = dev_any(c.w1, c.w_dtype), dev_any(c.w2, c.w_dtype)
        d["w1_scale"] = d["w2_scale"] = None
    if c.topk_ids is not None:
        d["topk_ids"] = dev_i32(c.topk_ids)
        d["topk_weights"] = dev_f32(c.topk_weights)
    d["expert_map"] = dev_i32(c.expert_map) if c.expert_map is not None else None
    return d


TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
