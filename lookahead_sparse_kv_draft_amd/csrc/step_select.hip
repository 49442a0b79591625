// The decode step's first launch carrying another state's selection (OasisKV
// explainer, Figure 8: a layer's prediction, selection and transfer proceed
// while later layers compute): the selection and diff of the previous layer
// (or of the last layer's previous step) run as leading workgroups of this
// layer's attention + scoring launch, which is bandwidth-bound and does not
// read what they write.  The step's second launch is then the attention's
// split combine alone.  The kernel is in step_kernel.h.
#include "attn_combine.h"
#include "step_kernel.h"

namespace oasis {

bool attn_score_select_available(const Ctx& c) {
  return attn_and_score_fused_available(c) && c.attn_waves == 2 && c.s.head_dim == 128 && select_wg_available(c);
}

hipError_t launch_attn_score_select(const Ctx& c, const void* q, const void* pool, const int32_t* attend,
                                    const int32_t* n_attend, const int32_t* ctx_attn, float* out, void* ws,
                                    const void* meta, const int32_t* ctx_score, float* scores, const SelectJob* job,
                                    hipStream_t st, const StepGather& g) {
  if (!attn_score_select_available(c)) return hipErrorInvalidValue;
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  const int kpt = (c.s.max_blocks + 127) / 128;  // keys per thread of a 128-thread selecting workgroup
  if (kpt <= 4)
    return as_d<128, 4>(c, q, pool, nullptr, nullptr, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta,
                        ctx_score, scores, g, job, st);
  if (kpt <= 16)
    return as_d<128, 16>(c, q, pool, nullptr, nullptr, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta,
                         ctx_score, scores, g, job, st);
  return as_d<128, 64>(c, q, pool, nullptr, nullptr, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta,
                       ctx_score, scores, g, job, st);
}

}  // namespace oasis
