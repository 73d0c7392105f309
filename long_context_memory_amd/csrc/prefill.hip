// Blocked prefill attention.
#include "msa_internal.h"

namespace msa {

hipError_t launch_prefill_vector(const Bank& bk, const void* q_rot, int n_q, int h_q,
                                 const int32_t* ids, int k, int block, const AttnSources& src,
                                 const void* k_loc, const void* v_loc, int L_loc, int splits,
                                 float* part, float* out, hipStream_t s);

hipError_t launch_prefill(const Bank& bk, const void* q_rot, int n_q, int h_q, const int32_t* ids,
                          int k, int block, const AttnSources& src, const void* k_loc,
                          const void* v_loc, int L_loc, int splits, float* part, float* out,
                          hipStream_t s) {
  return launch_prefill_vector(bk, q_rot, n_q, h_q, ids, k, block, src, k_loc, v_loc, L_loc,
                               splits, part, out, s);
}

}  // namespace msa
