// Host-only parameter checks and workspace sizing for librra.so.
// No HIP call is made here, so every rule can be exercised without a GPU.
#include <cmath>
#include <cstdint>

#include "rra.h"
#include "rra_internal.h"

namespace rra {

Shape shape_of(const rra_params_t& p) {
  Shape s;
  s.Bz = p.batch;
  s.H = p.num_heads;
  s.Hkv = p.num_kv_heads;
  s.L = p.seq_len;
  s.d = p.head_dim;
  s.S = p.stride;
  s.Bk = p.block;
  s.G = p.num_heads / (p.num_kv_heads > 0 ? p.num_kv_heads : 1);
  const int Sd = p.stride > 0 ? p.stride : 1;
  const int Bd = p.block > 0 ? p.block : 1;
  s.Ns = (p.seq_len + Sd - 1) / Sd;  // a last partial stride counts
  s.Nb = (p.seq_len + Bd - 1) / Bd;  // ceil(L / Bk), §2.1
  s.causal = p.causal != 0;
  s.r = p.block / (p.stride > 0 ? p.stride : 1);
  s.scale = (p.sm_scale > 0.0f) ? p.sm_scale : 1.0f / std::sqrt(static_cast<float>(p.head_dim));
  const int S = p.stride > 0 ? p.stride : 1;
  switch (p.rr_mode) {
    case RRA_RR_LAYER: s.rr_step = 0; s.rr_shift = p.rr_layer % S; break;
    case RRA_RR_HYBRID: s.rr_step = 1; s.rr_shift = p.rr_layer % S; break;
    case RRA_RR_NONE: s.rr_step = 0; s.rr_shift = p.rr_offset; break;
    default: s.rr_step = 1; s.rr_shift = 0; break;  // RRA_RR_HEAD
  }
  return s;
}

size_t kagg_bytes(const Shape& s) {
  return static_cast<size_t>(s.Bz) * s.Hkv * s.Ns * s.d * 2;
}

size_t score_bytes(const Shape& s) {
  return static_cast<size_t>(s.Bz) * s.H * s.Nb * s.Nb * 4;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace rra

extern "C" {

int rra_abi_version(void) { return RRA_ABI_VERSION; }

const char* rra_status_str(rra_status_t status) {
  switch (status) {
    case RRA_OK: return "RRA_OK";
    case RRA_ERR_INVALID_ARG: return "RRA_ERR_INVALID_ARG: invalid parameter or pointer";
    case RRA_ERR_UNSUPPORTED: return "RRA_ERR_UNSUPPORTED: shape or option not supported by this library";
    case RRA_ERR_WORKSPACE: return "RRA_ERR_WORKSPACE: workspace missing or too small";
    case RRA_ERR_HIP: return "RRA_ERR_HIP: HIP runtime error";
  }
  return "RRA_ERR_UNKNOWN";
}

rra_status_t rra_validate(const rra_params_t* p) {
  if (p == nullptr) return RRA_ERR_INVALID_ARG;
  // batch == 0 or seq_len == 0 is a valid empty problem (entry points do nothing).
  if (p->batch < 0 || p->seq_len < 0 || p->num_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 ||
      p->stride < 1 || p->block < 1)
    return RRA_ERR_INVALID_ARG;
  if (p->num_heads % p->num_kv_heads != 0) return RRA_ERR_INVALID_ARG;
  if (!(p->tau > 0.0f) || !(p->tau <= 1.0f)) return RRA_ERR_INVALID_ARG;  // also rejects NaN
  if (!std::isfinite(p->sm_scale)) return RRA_ERR_INVALID_ARG;
  if (p->protect_last != 0 && p->protect_last != 1) return RRA_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return RRA_ERR_INVALID_ARG;
  if (p->block % p->stride != 0) return RRA_ERR_INVALID_ARG;  // a block holds whole strides
  if (p->rr_mode < RRA_RR_HEAD || p->rr_mode > RRA_RR_NONE) return RRA_ERR_INVALID_ARG;
  if (p->rr_layer < 0 || p->rr_offset < 0 || p->rr_offset >= p->stride) return RRA_ERR_INVALID_ARG;
  // Shapes the kernels are built for.
  if (p->head_dim != 64 && p->head_dim != 128) return RRA_ERR_UNSUPPORTED;
  if (p->block != 64 && p->block != 128) return RRA_ERR_UNSUPPORTED;
  const int r = p->block / p->stride;
  if (r > 32) return RRA_ERR_UNSUPPORTED;  // strides per block must fit one 32-wide MFMA tile
  const int64_t nb = (static_cast<int64_t>(p->seq_len) + p->block - 1) / p->block;
  if (nb > rra::kMaxBlocks) return RRA_ERR_UNSUPPORTED;
  const int64_t elems_q = static_cast<int64_t>(p->batch) * p->num_heads * p->seq_len * p->head_dim;
  if (elems_q > (int64_t(1) << 40)) return RRA_ERR_UNSUPPORTED;
  const int64_t strides = static_cast<int64_t>(p->batch) * p->num_kv_heads * ((p->seq_len + p->stride - 1) / p->stride);
  if (strides >= (int64_t(1) << 31)) return RRA_ERR_UNSUPPORTED;
  return RRA_OK;
}

rra_status_t rra_estimate_workspace_size(const rra_params_t* p, size_t* bytes) {
  if (bytes == nullptr) return RRA_ERR_INVALID_ARG;
  rra_status_t st = rra_validate(p);
  if (st != RRA_OK) return st;
  const rra::Shape s = rra::shape_of(*p);
  *bytes = rra::align_up(rra::kagg_bytes(s), 256) + rra::align_up(rra::score_bytes(s), 256);
  return RRA_OK;
}

rra_status_t rra_attn_workspace_size(const rra_params_t* p, size_t* bytes) {
  if (bytes == nullptr) return RRA_ERR_INVALID_ARG;
  rra_status_t st = rra_validate(p);
  if (st != RRA_OK) return st;
  *bytes = rra::kSchedBytes;
  return RRA_OK;
}

}  // extern "C"
