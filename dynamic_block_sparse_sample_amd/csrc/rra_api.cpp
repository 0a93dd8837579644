// C ABI of librra.so: argument checks, workspace carving and kernel launches.
// Every entry point validates first and enqueues nothing on failure; all work
// is asynchronous on the caller's stream.
#include <cstdint>

#include "rra.h"
#include "rra_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }

rra_status_t hip_status(int err) { return err == 0 ? RRA_OK : RRA_ERR_HIP; }

bool empty_problem(const rra_params_t* p) { return p->batch == 0 || p->seq_len == 0; }

rra_status_t check(const rra_params_t* p) { return rra_validate(p); }

// The optional schedule workspace of the attention calls: nullptr, or at
// least kSchedBytes, 16-byte aligned.
rra_status_t sched_of(void* workspace, size_t workspace_bytes, uint32_t** sched) {
  *sched = nullptr;
  if (workspace == nullptr) return RRA_OK;
  if (!aligned16(workspace) || workspace_bytes < rra::kSchedBytes) return RRA_ERR_WORKSPACE;
  *sched = static_cast<uint32_t*>(workspace);
  return RRA_OK;
}

}  // namespace

extern "C" {

rra_status_t rra_cast_f32_to_bf16(const float* src, void* dst_bf16, int64_t n, void* stream) {
  if (n < 0) return RRA_ERR_INVALID_ARG;
  if (n == 0) return RRA_OK;
  if (!ok_ptr(src) || !ok_ptr(dst_bf16)) return RRA_ERR_INVALID_ARG;
  return hip_status(rra::launch_cast_f32_bf16(src, static_cast<uint16_t*>(dst_bf16), n, stream));
}

rra_status_t rra_stride_aggregate(const rra_params_t* p, const void* k, void* kagg, void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(k) || !ok_ptr(kagg)) return RRA_ERR_INVALID_ARG;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_stride_aggregate(s, static_cast<const uint16_t*>(k),
                                                 static_cast<uint16_t*>(kagg), stream));
}

rra_status_t rra_block_scores(const rra_params_t* p, const void* q, const void* kagg, float* score,
                              void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(q) || !ok_ptr(kagg) || !ok_ptr(score)) return RRA_ERR_INVALID_ARG;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_block_scores(s, static_cast<const uint16_t*>(q),
                                             static_cast<const uint16_t*>(kagg), score, stream));
}

rra_status_t rra_top_tau(const rra_params_t* p, const float* score, uint8_t* mask, int32_t* idx,
                         int32_t* cnt, void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(score) || mask == nullptr || !ok_ptr(idx) || !ok_ptr(cnt)) return RRA_ERR_INVALID_ARG;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_top_tau(s, p->tau, p->protect_last, score, mask, idx, cnt, stream));
}

rra_status_t rra_estimate(const rra_params_t* p, const void* q, const void* k, void* workspace,
                          size_t workspace_bytes, uint8_t* mask, int32_t* idx, int32_t* cnt,
                          float* score, void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || mask == nullptr || !ok_ptr(idx) || !ok_ptr(cnt)) return RRA_ERR_INVALID_ARG;
  if (score != nullptr && !aligned16(score)) return RRA_ERR_INVALID_ARG;
  size_t need = 0;
  st = rra_estimate_workspace_size(p, &need);
  if (st != RRA_OK) return st;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return RRA_ERR_WORKSPACE;
  const rra::Shape s = rra::shape_of(*p);
  uint16_t* kagg = static_cast<uint16_t*>(workspace);
  float* sc = score;
  if (sc == nullptr)
    sc = reinterpret_cast<float*>(static_cast<char*>(workspace) + rra::align_up(rra::kagg_bytes(s), 256));
  int err = rra::launch_stride_aggregate(s, static_cast<const uint16_t*>(k), kagg, stream);
  if (err == 0) err = rra::launch_block_scores(s, static_cast<const uint16_t*>(q), kagg, sc, stream);
  if (err == 0) err = rra::launch_top_tau(s, p->tau, p->protect_last, sc, mask, idx, cnt, stream);
  return hip_status(err);
}

rra_status_t rra_xattn_block_scores(const rra_params_t* p, const void* q, const void* k, float* score,
                                    void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  // Built for whole blocks, causal attention and (Bk, S) in {(128, 16), (128, 8), (128, 4), (64, 8), (64, 4)}.
  const bool shape_ok = (p->seq_len % p->block == 0) && p->causal == 1 &&
                        ((p->block == 128 && (p->stride == 16 || p->stride == 8 || p->stride == 4)) ||
                         (p->block == 64 && (p->stride == 8 || p->stride == 4)));
  if (!shape_ok) return RRA_ERR_UNSUPPORTED;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(score)) return RRA_ERR_INVALID_ARG;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_xattn_scores(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                             score, stream));
}

rra_status_t rra_block_mass(const rra_params_t* p, const void* q, const void* k, float* mass, void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(mass)) return RRA_ERR_INVALID_ARG;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_block_mass(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           mass, stream));
}

rra_status_t rra_sparse_attn(const rra_params_t* p, const void* q, const void* k, const void* v,
                             const int32_t* idx, const int32_t* cnt, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(idx) || !ok_ptr(cnt) || !ok_ptr(out))
    return RRA_ERR_INVALID_ARG;
  uint32_t* sched = nullptr;
  st = sched_of(workspace, workspace_bytes, &sched);
  if (st != RRA_OK) return st;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_flash_attn(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), idx, cnt,
                                           static_cast<uint16_t*>(out), sched, stream));
}

rra_status_t rra_dense_attn(const rra_params_t* p, const void* q, const void* k, const void* v, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  rra_status_t st = check(p);
  if (st != RRA_OK) return st;
  if (empty_problem(p)) return RRA_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(out)) return RRA_ERR_INVALID_ARG;
  uint32_t* sched = nullptr;
  st = sched_of(workspace, workspace_bytes, &sched);
  if (st != RRA_OK) return st;
  const rra::Shape s = rra::shape_of(*p);
  return hip_status(rra::launch_flash_attn(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), nullptr, nullptr,
                                           static_cast<uint16_t*>(out), sched, stream));
}

}  // extern "C"
