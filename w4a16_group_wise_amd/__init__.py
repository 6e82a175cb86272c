"""W4A16 group-wise quantization core for AMD gfx950 (MI355X).

Thin Python binding over libw4a16q.so (hand-written HIP kernels behind a C ABI, declared in
include/w4a16q.h).  The functions here only check tensor metadata, allocate outputs with
torch and pass raw device pointers plus the current HIP stream; every step of the
computation runs in the library's kernels.  There is no CPU fallback: if the library is
missing the calls raise.

Entry points (same names as the C ABI):
  quant_hessian, quant_scale_search, quant_pack, lsq_fwd, lsq_bwd, lsq_adam_step, w4a16_gemm, w4a16_gemm_dq,
  w4a16_gemv_grouped (and GemvGroupPlan, the same call with its problem table marshalled once),
  the per-channel variants quant_scale_search_pc, quant_pack_pc, lsq_fwd_pc, lsq_bwd_pc,
  w4a16_gemm_pc, the joint objective quant_joint_objective / quant_joint_refine, and the GPTQ
  error feedback quant_gptq
"""
from ._lib import (LIB_PATH, W4Q_EALIGN, W4Q_EHIP, W4Q_EINVAL, W4Q_ESHAPE, W4Q_EUNSUPPORTED,
                   W4Q_GROUP, W4Q_OK, W4QError, lib, status_string, version)
from .ops import (GemvGroupPlan, lsq_adam_step, lsq_bwd, lsq_bwd_pc, lsq_fwd, lsq_fwd_pc, probe_mfma_bf16,
                  probe_mfma_f64, probe_read, quant_gptq, quant_hessian, quant_joint_objective, quant_joint_refine, quant_pack,
                  quant_pack_pc, quant_scale_search, quant_scale_search_pc, w4a16_gemm, w4a16_gemm_dq,
                  w4a16_gemm_pc, w4a16_gemv_grouped, workspace_size)

__all__ = [
    "quant_hessian", "quant_scale_search", "quant_pack", "lsq_fwd", "lsq_bwd", "lsq_adam_step", "w4a16_gemm",
    "w4a16_gemm_dq",
    "w4a16_gemv_grouped", "GemvGroupPlan", "workspace_size",
    "quant_scale_search_pc", "quant_pack_pc", "lsq_fwd_pc", "lsq_bwd_pc", "w4a16_gemm_pc",
    "quant_joint_objective", "quant_joint_refine", "quant_gptq", "probe_read", "probe_mfma_bf16", "probe_mfma_f64",
    "W4QError", "lib", "LIB_PATH", "status_string", "version", "W4Q_GROUP", "W4Q_OK",
    "W4Q_EINVAL", "W4Q_ESHAPE", "W4Q_EALIGN", "W4Q_EUNSUPPORTED", "W4Q_EHIP",
]
