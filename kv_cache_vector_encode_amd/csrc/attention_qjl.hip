// Scores and fused decode attention over QJL keys (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv,
// TurboQuantCompressorV2.asymmetric_attention_scores): the kernels of attention_impl.h built with
// the sketch term, in a translation unit of their own so the two kernel sets compile in parallel.
#include "attention_impl.h"

namespace tq {

hipError_t launch_attention_qjl(const tq_attn_params* p, const Codebook& ck, const Codebook& cv, const Rotation& rk,
                                const Rotation& rv, float* scores, bool scores_only, const AttnLayout& lay,
                                hipStream_t st) {
  switch (rk.d) {
    case 64: return attn_bk<64, true>(p, ck, cv, rk, rv, scores, scores_only, lay, st);
    case 128: return attn_bk<128, true>(p, ck, cv, rk, rv, scores, scores_only, lay, st);
    default: return attn_bk<256, true>(p, ck, cv, rk, rv, scores, scores_only, lay, st);
  }
}

int attn_resident_waves_qjl(const tq_attn_params* p, int d, int bk, int bv, int device) {
  switch (d) {
    case 64: return attn_resident<64, true>(p, bk, bv, device);
    case 128: return attn_resident<128, true>(p, bk, bv, device);
    default: return attn_resident<256, true>(p, bk, bv, device);
  }
}

}  // namespace tq
