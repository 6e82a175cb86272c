"""Helpers for the GPU parity tests: numpy <-> device tensors and the parity criteria."""
import numpy as np
import torch

TIE_REL = 1e-6     # oracle near-tie window for the chosen candidate index
OBJ_REL = 1e-5     # objectives
H_REL = 1e-5       # Hessian entries, relative to sqrt(H_ii H_jj)
GEMM_REL = 1e-3    # W4A16 outputs, relative to sum |x * w_hat|
LSQ_REL = 1e-4     # step-size gradient


def dev_f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def dev_bf16(bits, dev):
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).to(dev).view(torch.bfloat16)


def host_bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f16_bits_to_np(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_np(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_hessian(h_gpu, h_ref, diag_ref=None):
    """|H - H_ref| <= H_REL * sqrt(H_ii H_jj) for fp64 reference entries."""
    h_gpu = np.asarray(h_gpu, dtype=np.float64)
    if diag_ref is None:
        d = np.diag(h_ref)
        bound = H_REL * np.sqrt(np.outer(d, d)) + 1e-30
    else:
        bound = H_REL * diag_ref + 1e-30
    err = np.abs(h_gpu - h_ref)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} Hessian entries out of tolerance; worst ratio {np.max(err / bound):.3g}"
    return float(np.max(err / bound))


def check_search(idx_g, scale_g, obj_g, idx_o, scale_o, obj_o, obj_all_o, cand_fn):
    """Exact index except oracle near-ties; scale = candidate at the GPU index; obj 1e-5 rel.

    cand_fn(flat_i, k) -> the oracle candidate scale of group flat_i at index k.
    """
    idx_g = idx_g.reshape(-1).astype(np.int64)
    idx_o = idx_o.reshape(-1).astype(np.int64)
    scale_g = scale_g.reshape(-1)
    obj_g = obj_g.reshape(-1).astype(np.float64)
    obj_o = obj_o.reshape(-1)
    oa = obj_all_o.reshape(idx_o.shape[0], -1)
    n_tie = 0
    for i in np.nonzero(idx_g != idx_o)[0]:
        best = oa[i].min()
        srt = np.sort(oa[i])
        near = srt[1] <= best * (1 + TIE_REL) if srt.shape[0] > 1 else False
        assert near and oa[i, idx_g[i]] <= best * (1 + TIE_REL), (
            f"group {i}: gpu idx {idx_g[i]} (obj {oa[i, idx_g[i]]!r}) vs oracle {idx_o[i]} "
            f"(obj {best!r})")
        n_tie += 1
    want_scale = np.array([cand_fn(i, k) if k != idx_o[i] else scale_o.reshape(-1)[i]
                           for i, k in enumerate(idx_g)], dtype=np.float32) if n_tie else scale_o.reshape(-1)
    assert np.array_equal(scale_g, want_scale)
    ref = oa[np.arange(oa.shape[0]), idx_g]
    err = np.abs(obj_g - ref)
    assert np.all(err <= OBJ_REL * ref + 1e-30), f"obj worst rel {np.max(err / (ref + 1e-30)):.3g}"
    return n_tie


def check_gemm(y_gpu, y_ref, yabs, bf16_out=False):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    bound = GEMM_REL * yabs
    if bf16_out:
        # half an ulp of bf16 at the reference magnitude
        e = np.floor(np.log2(np.maximum(np.abs(y_ref), 1e-38)))
        bound = bound + 0.5 * np.exp2(e - 7)
    err = np.abs(y_gpu - y_ref)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs out of tolerance; worst ratio {np.max(err / (bound + 1e-300)):.3g}"
    rel2 = np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    return float(np.max(err / (bound + 1e-300))), float(rel2)


def search_bound(w, h, alpha, cand_fn):
    """B[r][g][k] = |e|^T |H_gg| |e| for every group and candidate (the scale of a pass-1 score's
    rounding error), e = w - d_k * code(w, d_k) with the oracle's candidate steps cand_fn(i, k)
    (flat group index i) and nearest-even codes clamped to [-8, 7]."""
    d_out, d_in = w.shape
    G, K = d_in // 32, alpha.shape[0]
    wg = w.reshape(d_out, G, 32).astype(np.float64)
    out = np.empty((d_out, G, K))
    for g in range(G):
        ha = np.abs(np.asarray(h, dtype=np.float64)[32 * g:32 * g + 32, 32 * g:32 * g + 32])
        d = np.array([[cand_fn(r * G + g, k) for k in range(K)] for r in range(d_out)])  # [r][k]
        safe = np.where(d == 0, 1.0, d)
        q = np.clip(np.rint(wg[:, g, None, :] / safe[:, :, None]), -8, 7)
        e = np.abs(wg[:, g, None, :] - d[:, :, None] * q)
        out[:, g, :] = np.einsum("rki,ij,rkj->rk", e, ha, e)
    return out
